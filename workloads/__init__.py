"""Seeded synthetic inputs for the W4A16 AWQ linear layer.

This module only draws numbers: it holds none of the quantizer's or the
layer's arithmetic, and both the CPU oracle's tests and the HIP path take
their inputs from here.

The pages measure trained Llama/Mistral/Qwen checkpoints and calibrate on
text corpora ("Optimization Awq", sections "Benchmarks de desempenho" and
"Calibração personalizada"); none of those is available, so these seeded
draws stand in for them.  Shapes are Llama-7B (hidden 4096, MLP 11008) and
70B-like (8192 / 28672) linears.  Recipe:

* W[N, K]: fp32 standard normal / sqrt(K), optionally plus one per-row mean
  offset mu_n ~ U(-sigma/2, sigma/2) (sigma = 1/sqrt(K)), cast to fp16.
* X[M, K]: fp32 standard normal; round(0.01 K) input channels, drawn without
  replacement, are multiplied by 20 (activation outliers, the same channels in
  every row); cast to fp16.
* Seeds: ``numpy.random.default_rng([seed, cfg, layer])`` for W and
  ``default_rng([seed, cfg, layer, M, 1])`` for X.
"""
from __future__ import annotations

import numpy as np

# (name, K, N) of the seven linears of one Llama-7B decoder block.
LLAMA7B_BLOCK = (
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 4096),
    ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 4096, 11008),
    ("up_proj", 4096, 11008),
    ("down_proj", 11008, 4096),
)

# (name, K, N) of the two 70B-shaped MLP linears used for prefill.
LLAMA70B_MLP = (
    ("up_proj_70b", 8192, 28672),
    ("down_proj_70b", 28672, 8192),
)

OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 20.0


def weight(N: int, K: int, cfg: int, layer: int, seed: int = 0, row_offset: bool = False) -> np.ndarray:
    """fp16 [N, K] weight drawn from N(0, 1/K), optionally with per-row mean offsets."""
    rng = np.random.default_rng([seed, cfg, layer])
    sigma = np.float32(1.0 / np.sqrt(K))
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= sigma
    if row_offset:
        mu = rng.uniform(-0.5, 0.5, size=(N, 1)).astype(np.float32) * sigma
        W += mu
    return W.astype(np.float16)


def outlier_channels(K: int, rng: np.random.Generator) -> np.ndarray:
    count = int(round(OUTLIER_FRACTION * K))
    return np.sort(rng.choice(K, size=count, replace=False))


def activations(M: int, K: int, cfg: int, layer: int, seed: int = 0) -> np.ndarray:
    """fp16 [M, K] activations: N(0, 1) with 1% of the channels scaled by 20."""
    rng = np.random.default_rng([seed, cfg, layer, M, 1])
    X = rng.standard_normal((M, K), dtype=np.float32)
    idx = outlier_channels(K, rng)
    X[:, idx] *= np.float32(OUTLIER_GAIN)
    return X.astype(np.float16)


def adversarial_weight(N: int, K: int, g: int, seed: int = 0) -> np.ndarray:
    """fp16 [N, K] weight whose groups cycle through awkward cases.

    Group kinds, chosen per (row, group) from the seed: ordinary Gaussian;
    all zeros; one constant value; all positive (the range excludes 0);
    all negative; values on an exact half-step grid (rounding ties); fp16
    subnormals only; a mix of +0.0 and -0.0 with one nonzero value; a few
    large values (|w| up to 60000) among small ones.
    """
    rng = np.random.default_rng([seed, 0xAD, N, K, g])
    G = K // g
    W = np.empty((N, G, g), dtype=np.float32)
    kinds = rng.integers(0, 9, size=(N, G))
    base = rng.standard_normal((N, G, g), dtype=np.float32) / np.float32(np.sqrt(K))
    for n in range(N):
        for j in range(G):
            k = kinds[n, j]
            b = base[n, j]
            if k == 0:
                v = b
            elif k == 1:
                v = np.zeros(g, np.float32)
            elif k == 2:
                v = np.full(g, b[0], np.float32)
            elif k == 3:
                v = np.abs(b) + np.float32(0.25)
            elif k == 4:
                v = -np.abs(b) - np.float32(0.125)
            elif k == 5:
                # multiples of 1/32 in [-0.25, 0.6875]: with s = 1/16 every odd
                # multiple sits exactly halfway between two grid points.
                v = rng.integers(-8, 23, size=g).astype(np.float32) / np.float32(32)
            elif k == 6:
                v = rng.integers(-1023, 1024, size=g).astype(np.float32) * np.float32(2.0 ** -24)
            elif k == 7:
                v = np.where(rng.integers(0, 2, size=g) == 1, np.float32(0.0), np.float32(-0.0))
                v[rng.integers(0, g)] = b[0]
            else:
                v = b.copy()
                v[rng.integers(0, g, size=2)] = rng.uniform(-60000, 60000, size=2).astype(np.float32)
            W[n, j] = v
    return W.reshape(N, K).astype(np.float16)
