"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds none of the layer's arithmetic: it only draws the fp16
activations and weights that both sides consume byte-for-byte.

Recipe (the pages measure on real checkpoints and wikitext2, which are not
used here; these tensors stand in for them in shape and value range):
  * generator: numpy PCG64 ``default_rng`` with sub-streams
      X <- [seed, 0, K],  outlier columns <- [seed, 1, K],
      W <- [seed, 2, N, K],  stacked-layer weights <- [seed, 3, layer, j];
  * X: float32 N(0, 1); round(K/100) whole columns (channel outliers, the
    same for every row) multiplied by 20; cast to fp16 (round to nearest even).
    Rows are drawn in order, so the first M rows of a larger draw equal a
    draw of M rows: an M sweep is nested;
  * W: std * N(0, 1) in float32, cast to fp16, shape [N, K] (out x in, as
    nn.Linear stores it); std = 0.02 for the operator sweeps, 1/sqrt(K) for
    the stacked decoder layers (unit gain, so activations stay in fp16 range).
"""
from __future__ import annotations

import numpy as np

OUTLIER_SCALE = 20.0


def outlier_columns(K: int, seed: int = 0) -> np.ndarray:
    count = int(np.floor(K / 100.0 + 0.5))
    rng = np.random.default_rng([seed, 1, K])
    return np.sort(rng.choice(K, count, replace=False))


def activations(M: int, K: int, seed: int = 0, outliers: bool = True) -> np.ndarray:
    """fp16 [M, K]."""
    rng = np.random.default_rng([seed, 0, K])
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        x[:, outlier_columns(K, seed)] *= np.float32(OUTLIER_SCALE)
    return x.astype(np.float16)


def weights(N: int, K: int, seed: int = 0, std: float = 0.02) -> np.ndarray:
    """fp16 [N, K]."""
    rng = np.random.default_rng([seed, 2, N, K])
    return (np.float32(std) * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float16)


def layer_weights(layer: int, j: int, N: int, K: int, seed: int = 0) -> np.ndarray:
    """fp16 [N, K] for GEMM j of decoder layer `layer`, std 1/sqrt(K)."""
    rng = np.random.default_rng([seed, 3, layer, j])
    std = np.float32(1.0 / np.sqrt(K))
    return (std * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float16)


# The operator workloads: (name, mode, N, K, group sizes, M values).
M_SWEEP = (1, 128, 1024, 4096, 8192)
WORKLOADS = {
    "w8a8_pc_small": dict(bits=8, N=512, K=1024, group_sizes=(0,), M=(64,)),
    "w8a8_pc": dict(bits=8, N=10240, K=2560, group_sizes=(0,), M=M_SWEEP),
    "w8a8_pg": dict(bits=8, N=2560, K=10240, group_sizes=(64, 128), M=M_SWEEP),
    "w4a8_pc": dict(bits=4, N=10240, K=2560, group_sizes=(0,), M=M_SWEEP),
    "w4a8_pg": dict(bits=4, N=2560, K=10240, group_sizes=(64, 128), M=M_SWEEP),
}

# 8B-class decoder layer: (name, N, K, column offset of its input in the
# previous GEMM's output, ldx of that input).  QKV reads the layer input;
# O reads the first 4096 columns of the QKV output; gate+up reads O's output;
# down reads the first 12288 columns of gate+up's output.
DECODER_LAYER = (
    ("qkv", 6144, 4096),
    ("o", 4096, 4096),
    ("gate_up", 24576, 4096),
    ("down", 4096, 12288),
)
DECODER_LAYERS = 36
DECODER_TOKENS = 4096
