"""Seeded synthetic inputs for the bitmap SpMM path.

This module produces the dense weight matrix W, the keep mask and the
activations X that both the CPU oracle and the GPU path consume.  It holds
none of the method's arithmetic: no bitmap packing, no popcount, no product,
no quantisation.  Every generator takes a ``numpy.random.Generator`` so that a
caller can reproduce an input from its seed tuple alone.

Workload recipes (stand-ins for the pages' model-derived shape sets, which
use trained OPT/LLaMA weights that are not available here):

* W ~ N(0, 0.02) in fp64, rounded to fp16 (round-to-nearest-even).
* Unstructured masks: i.i.d. Bernoulli keep, magnitude pruning (drop the
  floor(s*M*K) smallest |w|, ties broken by linear index), or per-row keep
  probabilities drawn from Beta(2, 2) and rescaled to a target mean.
* X ~ N(0, 1) in fp64, rounded to fp16, stored as [N][K] (one row per token).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "seed_rng",
    "weight_normal",
    "weight_dyadic",
    "weight_int4_exact",
    "activations_normal",
    "activations_small_int",
    "mask_bernoulli",
    "mask_magnitude",
    "mask_beta_rows",
    "LAYERS_OPT13B",
    "LAYERS_PREFILL",
    "CONFIG_NAMES",
    "config_case",
]

# Layer shapes (M, K) of an OPT-13B decoder block (hidden 5120, FFN 20480).
LAYERS_OPT13B = {
    "qkv": (15360, 5120),
    "attn_out": (5120, 5120),
    "ffn_up": (20480, 5120),
    "ffn_down": (5120, 20480),
}
# Llama-7B-shaped FFN projections (hidden 4096, FFN 11008).
LAYERS_PREFILL = {
    "up": (11008, 4096),
    "down": (4096, 11008),
}
CONFIG_NAMES = {1: "tiny", 2: "opt13b_decode", 3: "sparsity_sweep", 4: "prefill", 5: "int4"}


def seed_rng(config_id: int, layer_id: int = 0, tensor_id: int = 0) -> np.random.Generator:
    """Generator for one tensor of one layer of one workload.

    The tiny workload (id 1) uses plain seed 0 for its first tensor; every other
    tensor uses the tuple (0, config_id, layer_id, tensor_id).
    """
    if config_id == 1 and layer_id == 0 and tensor_id == 0:
        return np.random.default_rng(0)
    return np.random.default_rng((0, config_id, layer_id, tensor_id))


def weight_normal(M: int, K: int, rng: np.random.Generator, sigma: float = 0.02) -> np.ndarray:
    """Dense fp16 weight [M][K] with entries N(0, sigma^2), sampled in fp64."""
    return rng.normal(0.0, sigma, size=(M, K)).astype(np.float16)


def weight_dyadic(M: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """Dense fp16 weight with entries k/8, |k| <= 16 (exactly representable).

    Products with small-integer activations and their partial sums stay exact
    in fp32, so any summation order gives the same bits.
    """
    return (rng.integers(-16, 17, size=(M, K)).astype(np.float64) / 8.0).astype(np.float16)


def weight_int4_exact(M: int, K: int, rng: np.random.Generator, mask: np.ndarray) -> np.ndarray:
    """fp16 weight whose per-row INT4 quantisation is exact.

    Row m holds q * 2^e_m with integer q in [-7, 7] and one kept entry equal
    to +-7 * 2^e_m, so the row's largest kept magnitude over 7 is the power of
    two 2^e_m and every kept entry is an exact multiple of it.
    """
    e = rng.integers(-9, -3, size=M)
    q = rng.integers(-7, 8, size=(M, K)).astype(np.float64)
    for m in range(M):
        kept = np.flatnonzero(mask[m])
        if kept.size:
            q[m, kept[rng.integers(kept.size)]] = 7.0 * (1 if rng.random() < 0.5 else -1)
    return (q * np.exp2(e)[:, None]).astype(np.float16)


def weight_int2_exact(M: int, K: int, rng: np.random.Generator, mask: np.ndarray) -> np.ndarray:
    """fp16 weight whose per-row 2-bit quantisation is exact.

    Row m holds q * 2^e_m with q in {-1, 0, 1} and one kept entry equal to
    +-2^e_m, so the row's largest kept magnitude is the power of two 2^e_m
    and every kept entry is an exact multiple of it.
    """
    e = rng.integers(-9, -3, size=M)
    q = rng.integers(-1, 2, size=(M, K)).astype(np.float64)
    for m in range(M):
        kept = np.flatnonzero(mask[m])
        if kept.size:
            q[m, kept[rng.integers(kept.size)]] = 1.0 if rng.random() < 0.5 else -1.0
    return (q * np.exp2(e)[:, None]).astype(np.float16)


def activations_normal(N: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """Activations X stored [N][K] fp16, entries N(0, 1) sampled in fp64."""
    return rng.normal(0.0, 1.0, size=(N, K)).astype(np.float16)


def activations_small_int(N: int, K: int, rng: np.random.Generator, lim: int = 3) -> np.ndarray:
    """Activations with integer entries in [-lim, lim] (exact in fp16)."""
    return rng.integers(-lim, lim + 1, size=(N, K)).astype(np.float16)


def mask_bernoulli(M: int, K: int, keep: float, rng: np.random.Generator) -> np.ndarray:
    """i.i.d. Bernoulli(keep) mask, bool [M][K]."""
    return rng.random(size=(M, K)) < keep


def mask_magnitude(W: np.ndarray, sparsity: float) -> np.ndarray:
    """Magnitude pruning: drop the floor(s*M*K) entries of smallest |w|.

    Ties are broken by linear (row-major) index: among equal magnitudes the
    earlier element is dropped first.  For fp16 input the sort key is the bit
    pattern with the sign cleared, which orders finite magnitudes exactly.
    """
    M, K = W.shape
    n_drop = int(np.floor(sparsity * M * K))
    if W.dtype == np.float16:
        key = W.reshape(-1).view(np.uint16) & np.uint16(0x7FFF)
    else:
        key = np.abs(W.reshape(-1).astype(np.float64))
    order = np.argsort(key, kind="stable")
    keep = np.ones(M * K, dtype=bool)
    keep[order[:n_drop]] = False
    return keep.reshape(M, K)


def mask_beta_rows(M: int, K: int, sparsity: float, rng: np.random.Generator,
                   a: float = 2.0, b: float = 2.0) -> np.ndarray:
    """Row-nonuniform unstructured mask.

    Each row r draws a keep probability p_r ~ Beta(a, b).  The p_r are scaled
    multiplicatively towards the target mean 1 - s and clipped to [0, 1],
    repeating the scale-and-clip step until the mean is within 1e-9 of the
    target; then each entry of row r is kept with probability p_r.
    """
    target = 1.0 - sparsity
    p = rng.beta(a, b, size=M)
    for _ in range(200):
        mean = p.mean()
        if abs(mean - target) < 1e-9 or mean == 0.0:
            break
        p = np.clip(p * (target / mean), 0.0, 1.0)
    return rng.random(size=(M, K)) < p[:, None]


def config_case(config_id: int, M: int, K: int, N: int, sparsity: float, layer_id: int = 0,
                exact: bool = False):
    """(W fp16 [M][K], mask bool [M][K], X fp16 [N][K]) for one workload case.

    Workload ids: 1 tiny (Bernoulli 0.5 keep), 2 OPT-13B decode layers and
    4 prefill layers (magnitude pruning), 3 sparsity sweep (Beta(2,2) rows),
    5 INT4 (magnitude pruning; quantisation happens in the encoder).
    ``exact`` swaps in dyadic W and small-integer X for bitwise comparisons.
    """
    rw = seed_rng(config_id, layer_id, 0)
    rm = seed_rng(config_id, layer_id, 1)
    rx = seed_rng(config_id, layer_id, 2 + N)
    W = weight_dyadic(M, K, rw) if exact else weight_normal(M, K, rw)
    if config_id == 1:
        mask = mask_bernoulli(M, K, 1.0 - sparsity, rm)
    elif config_id == 3:
        mask = mask_beta_rows(M, K, sparsity, rm)
    elif exact:
        mask = mask_bernoulli(M, K, 1.0 - sparsity, rm)
    else:
        mask = mask_magnitude(W, sparsity)
    X = activations_small_int(N, K, rx) if exact else activations_normal(N, K, rx)
    return W, mask, X
