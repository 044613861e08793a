"""Seeded synthetic inputs for the top-k workloads.

This module only draws numbers: it holds none of the selection method's
arithmetic, and both the oracle-side checks and the GPU-side tests and
benchmark take their inputs from here.

Distributions follow the Prof-K paper's synthetic study (section 5,
"Experimental Setup": Uniform, Standard Normal and heavy-tailed Pareto) and
its BatchTopK application (section 5, "Application": post-ReLU activations of
shape B x d_dict flattened).  The GPU.js Learn pages supply the small integer
rows (4,096 scores with heavy ties; 65,536 finer-grained scores).

Recipes (numpy ``Generator(PCG64(seed))``):

* ``scores_int``  int32 ``integers(lo, hi)``.
* ``normal_f32``  ``standard_normal(dtype=float32)``.
* ``pareto_signed``  Pareto type I, scale 1, shape 1.5, magnitudes
  ``(1 - U) ** (-1 / 1.5)`` in float64 rounded to float32, times an
  equiprobable sign.
* ``sorted_rows``  the same rows sorted ascending.
* ``planted``  float32 rows of +0.0 with ``m`` distinct positions per row
  (``choice(n, m, replace=False)``) set to 1.0.
* ``relu_bf16``  float32 ``standard_normal`` -> ``maximum(x, 0)`` (+0.0 for
  negatives) -> bf16 by round-to-nearest-even, returned as uint16 bits.
"""
from __future__ import annotations

import numpy as np

SEEDS = {"c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004, "c5": 1005}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def scores_int(rows: int, n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    return rng(seed).integers(lo, hi, size=(rows, n), dtype=np.int32)


def normal_f32(rows: int, n: int, seed: int) -> np.ndarray:
    g = rng(seed)
    return g.standard_normal(size=(rows, n), dtype=np.float32)


def pareto_signed(rows: int, n: int, seed: int, shape: float = 1.5) -> np.ndarray:
    g = rng(seed)
    u = g.random(size=(rows, n))
    mag = (1.0 - u) ** (-1.0 / shape)
    sign = np.where(g.random(size=(rows, n)) < 0.5, -1.0, 1.0)
    return (mag * sign).astype(np.float32)


def sorted_rows(x: np.ndarray) -> np.ndarray:
    return np.sort(x, axis=1)


def planted(rows: int, n: int, m: int, seed: int) -> np.ndarray:
    g = rng(seed)
    x = np.zeros((rows, n), dtype=np.float32)
    for r in range(rows):
        x[r, g.choice(n, m, replace=False)] = 1.0
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); finite inputs only."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def relu_bf16(rows: int, n: int, seed: int) -> np.ndarray:
    x = rng(seed).standard_normal(size=(rows, n), dtype=np.float32)
    np.maximum(x, np.float32(0.0), out=x)
    x[x == 0] = np.float32(0.0)          # +0.0, never -0.0
    return f32_to_bf16_bits(x)


def c2_seed(start: int = SEEDS["c2"], k: int = 10) -> int:
    """First seed >= start whose 65,536 scores have distinct k-th and (k+1)-th
    largest values (the counting bisection needs a gap there)."""
    s = start
    while True:
        x = scores_int(1, 65536, 0, 2 ** 24, s)[0]
        top = np.sort(x)[::-1]
        if top[k - 1] != top[k]:
            return s
        s += 1


def config(name: str, seed: int | None = None):
    """The five headline workloads.  Returns (array, dtype_name, k_list, meta).

    Array shapes: [rows, n]; bf16 is returned as uint16 bits.
    """
    if name == "c1":
        s = SEEDS["c1"] if seed is None else seed
        return scores_int(1, 4096, 0, 1000, s), "int32", [10], {"seed": s}
    if name == "c2":
        s = c2_seed() if seed is None else seed
        return scores_int(1, 65536, 0, 2 ** 24, s), "int32", [10], {"seed": s}
    if name == "c3":
        s = SEEDS["c3"] if seed is None else seed
        return normal_f32(1, 2 ** 28, s), "float32", [16, 64, 2048], {"seed": s}
    if name in ("c4v1", "c4v2", "c4v3"):
        s = SEEDS["c4"] if seed is None else seed
        if name == "c4v3":
            return planted(128, 2 ** 20, 64, s), "float32", [64], {"seed": s}
        x = pareto_signed(128, 2 ** 20, s)
        if name == "c4v2":
            x = sorted_rows(x)
        return x, "float32", [64], {"seed": s}
    if name == "c5":
        s = SEEDS["c5"] if seed is None else seed
        return relu_bf16(4096, 65536, s), "bf16", [131072], {"seed": s}
    raise KeyError(name)
