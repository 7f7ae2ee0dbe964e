"""Seeded synthetic inputs for the five workloads.

This module is shared by the tests, the benchmark and the smoke check.  It
holds only random-number recipes and shapes, none of the method's
arithmetic, and imports neither the oracle nor the product package.

Data come from NumPy's PCG64 generator (``np.random.default_rng(seed)``),
drawn as float32 and rounded to the 16-bit formats on the CPU with
round-to-nearest-even (NumPy for fp16, torch for bf16).  Arrays are returned
as raw bit patterns (uint16 / uint32 / int32) because every call on the path
is a bit copy whose result is compared bit for bit.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np

__all__ = [
    "map_offsets",
    "map_triples",
    "fp32_matrix",
    "fp16_matrix",
    "bf16_tensor",
    "bf16_operands",
    "bf16_bits",
    "FULL",
]

# Full sizes of the five workloads.
FULL = {
    "map": {"n": 65536},
    "fp32_transpose": {"rows": 4096, "cols": 4096},
    "fp16_transpose": {"rows": 8192, "cols": 8192},
    "bf16_convert": {"batch": 64, "rows": 4096, "cols": 128},
    "bf16_stage": {"m": 8192, "n": 8192, "k": 4096},
}


def map_offsets(n: int = 65536) -> np.ndarray:
    """int32 offsets 0..n-1."""
    return np.arange(n, dtype=np.int32)


def map_triples() -> List[Tuple[int, int, int]]:
    """Every (B, M, S) with B in 1..5, M in 0..4, S in B..7, lexicographic."""
    return [(B, M, S) for B in range(1, 6) for M in range(0, 5) for S in range(B, 8)]


def fp32_matrix(rows: int, cols: int, seed: int = 0) -> np.ndarray:
    """Uniform[-1, 1) float32, returned as uint32 bits."""
    rng = np.random.default_rng(seed)
    x = rng.random((rows, cols), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    return x.view(np.uint32)


def fp16_matrix(rows: int, cols: int, seed: int = 0) -> np.ndarray:
    """Normal(0, 1) drawn as float32, rounded to fp16, returned as uint16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32).astype(np.float16)
    return x.view(np.uint16)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_tensor(shape, seed: int = 0, lo: float = -4.0, hi: float = 4.0) -> np.ndarray:
    """Uniform[lo, hi) float32 rounded to bf16 (uint16 bits)."""
    rng = np.random.default_rng(seed)
    x = rng.random(tuple(shape), dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    return bf16_bits(x)


def bf16_operands(m: int, n: int, k: int, seed: int = 0, std: float = 0.02):
    """GEMM operands as bf16 bits: A[m][k] row-major, then B[k][n] column-major,
    which is the same memory as B^T[n][k] row-major.  Both are
    Normal(0, std), A drawn first."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((m, k), dtype=np.float32) * np.float32(std)
    bt = rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    return bf16_bits(a), bf16_bits(bt)
