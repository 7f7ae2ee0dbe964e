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
    "u8_matrix",
    "bf16_tensor",
    "bf16_operands",
    "bf16_bits",
    "index_pattern_device",
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


def u8_matrix(rows: int, cols: int, seed: int = 0) -> np.ndarray:
    """Uniform random bytes (an int8 / fp8 matrix as raw bits), uint8."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)


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


def index_pattern_device(shape, device, elem_bytes: int = 4):
    """A large input made on the GPU without a host copy: element
    (i0, ..., in) of a C-contiguous tensor of `shape` holds
    (7 * i0 + 13 * (i0 >> 12) + flat index inside the first dimension) mod
    2^(8*elem_bytes - 1), as int32 (elem_bytes 4) or int16 (elem_bytes 2); the
    second term keeps leading indices 2^15 apart (a 15-bit pattern repeats
    there under 7 * i0 alone) from holding the same values.  Every value is
    recomputable on the host from the element's coordinates, so sampled
    outputs of very large calls can be checked without generating the whole
    input twice.  No randomness: used where the input is too large for the
    seeded host generators."""
    import torch

    first = shape[0]
    inner = 1
    for d in shape[1:]:
        inner *= d
    mask = (1 << (8 * elem_bytes - 1)) - 1
    i0 = torch.arange(first, dtype=torch.int64, device=device)
    base = (i0 * 7 + (i0 >> 12) * 13).view(first, 1)
    flat = torch.arange(inner, dtype=torch.int64, device=device).view(1, inner)
    out_dtype = torch.int32 if elem_bytes == 4 else torch.int16
    out = torch.empty((first, inner), dtype=out_dtype, device=device)
    step = max(1, (1 << 26) // max(inner, 1))  # bound the int64 temporaries
    for b0 in range(0, first, step):
        out[b0:b0 + step] = ((base[b0:b0 + step] + flat) & mask).to(out_dtype)
    return out.view(*shape)


def index_pattern_host(shape, index, elem_bytes: int = 4) -> np.ndarray:
    """The values index_pattern_device puts at the given leading index
    (a sub-array of shape[1:]), as uint32 / uint16 bits."""
    inner = int(np.prod(shape[1:]))
    mask = (1 << (8 * elem_bytes - 1)) - 1
    i0 = int(index)
    v = (7 * i0 + 13 * (i0 >> 12) + np.arange(inner, dtype=np.int64)) & mask
    return v.astype(np.uint32 if elem_bytes == 4 else np.uint16).reshape(shape[1:])
