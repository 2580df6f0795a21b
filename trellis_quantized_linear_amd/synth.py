"""Seeded synthetic inputs for the EXL3 linear.

This module holds none of the method's arithmetic: it only draws random bits
and converts random reals to fp16/bf16 with numpy's and torch's own
round-to-nearest-even casts.  Both the HIP path and the CPU oracle take their
inputs from here, so each test and benchmark line can name its seeds.

Every tensor is returned as a numpy array of raw bit patterns (uint8 packed
words, uint16 fp16/bf16 values); callers move them to the device themselves.

Recipe (the pages' workloads are 27B-shaped layers served from trained
checkpoints; no checkpoint is present, so only the shapes are reproduced):
  * packed trellis words: uniform random bytes, so every 16-bit state is
    equally likely;
  * per-column scales: fp16 of U(0.5, 2);
  * sign vectors suh, svh: fair +-1 in fp16;
  * activations X: bf16 of N(0, sigma), sigma = 1 (0.5 for prompt prefill).
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

FP16_ONE = 0x3C00
FP16_MINUS_ONE = 0xBC00


def seed_for(*names) -> int:
    """A stable 63-bit seed from a tuple of names (config, member, tensor)."""
    h = hashlib.sha256("/".join(str(n) for n in names).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def rng_for(*names) -> np.random.Generator:
    return np.random.default_rng(seed_for(*names))


def words_nbytes(K: int, N: int, bits: int) -> int:
    return K * N * bits // 8


def gen_words(rng: np.random.Generator, K: int, N: int, bits: int) -> np.ndarray:
    """Uniform random packed words for a K x N weight (dense block-major)."""
    return rng.integers(0, 256, size=words_nbytes(K, N, bits), dtype=np.uint8)


def gen_scales(rng: np.random.Generator, n: int, lo: float = 0.5, hi: float = 2.0) -> np.ndarray:
    return rng.uniform(lo, hi, size=n).astype(np.float16).view(np.uint16)


def gen_signs(rng: np.random.Generator, n: int) -> np.ndarray:
    s = rng.integers(0, 2, size=n)
    return np.where(s == 1, FP16_MINUS_ONE, FP16_ONE).astype(np.uint16)


def gen_x(rng: np.random.Generator, M: int, K: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of N(0, sigma) [M, K] (torch's float32 -> bf16 cast)."""
    import torch
    x = rng.standard_normal(size=(M, K)).astype(np.float32) * np.float32(sigma)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclass
class LayerInputs:
    """One EXL3 weight's host-side inputs as raw bit patterns."""
    name: str
    K: int
    N: int
    bits: int
    words: np.ndarray    # uint8 [K*N*bits/8], block-major
    scales: np.ndarray   # uint16 fp16 [N]
    suh: np.ndarray      # uint16 fp16 [K]
    svh: np.ndarray      # uint16 fp16 [N]


def gen_layer(config: str, name: str, K: int, N: int, bits: int) -> LayerInputs:
    """A weight with every tensor drawn from its own named seed."""
    return LayerInputs(
        name=name, K=K, N=N, bits=bits,
        words=gen_words(rng_for(config, name, "words"), K, N, bits),
        scales=gen_scales(rng_for(config, name, "scales"), N),
        suh=gen_signs(rng_for(config, name, "suh"), K),
        svh=gen_signs(rng_for(config, name, "svh"), N),
    )


# The pages' 27B dense layer: hidden 5120, intermediate 17408, vocabulary
# 248,320 (head 5120 -> 248320), q 6144 and k/v 1024 columns.
HIDDEN = 5120
INTERMEDIATE = 17408
VOCAB = 248320
Q_COLS = 6144
KV_COLS = 1024
