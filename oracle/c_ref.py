"""ctypes binding of the plain C oracle (oracle/c/oracle_ref.c).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite
pins it against library routines and the pages' worked example, and the
benchmark's CPU-baseline leg times it.  The shared library is compiled with
gcc on first use (and by the build entry point), next to its source.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "oracle_ref.c")
LIB = os.path.join(HERE, "c", "liboracle_ref.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc -O2 (plain loops; no vector extensions asked for)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, SRC], check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.oref_swizzle.argtypes = [ctypes.c_uint32, i32, i32, i32]
        L.oref_swizzle.restype = ctypes.c_uint32
        L.oref_swizzle_map.argtypes = [vp, vp, i64, i32, i32, i32]
        L.oref_swizzle_map.restype = None
        L.oref_convert.argtypes = [vp, vp, i64, i64, i64, i32, i32]
        L.oref_convert.restype = ctypes.c_int
        L.oref_stage_operand.argtypes = [vp, vp, i64, i64, i32]
        L.oref_stage_operand.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def swizzle_map(x, B, M, S):
    """out[i] = Swizzle<B,M,S>(x[i]) on uint32 bit patterns ("CuTe Swizzle 学习手册", swizzle formula)."""
    if min(B, M) < 0 or B + M + abs(S) > 31:
        raise ValueError("need B, M >= 0 and B + M + |S| <= 31")
    x = np.ascontiguousarray(x, dtype=np.int32)
    out = np.empty_like(x)
    lib().oref_swizzle_map(_ptr(x), _ptr(out), x.size, B, M, S)
    return out


def convert_layout(a, threads: int = 1):
    """dst[b][c][r] = src[b][r][c] for a [batch, rows, cols] (or [rows, cols])
    array of 1-, 2- or 4-byte elements, as raw bits ("CUDA 013 - Swizzle 的工作原理",
    problem statement)."""
    a = np.ascontiguousarray(a)
    if a.itemsize not in (1, 2, 4) or a.ndim not in (2, 3):
        raise ValueError("1-, 2- or 4-byte elements, 2-D or 3-D")
    a3 = a.reshape((1,) + a.shape) if a.ndim == 2 else a
    b, r, c = a3.shape
    out = np.empty((b, c, r), dtype=a.dtype)
    if lib().oref_convert(_ptr(a3), _ptr(out), b, r, c, a.itemsize, threads) != 0:
        raise ValueError("oref_convert rejected its arguments")
    return out.reshape(c, r) if a.ndim == 2 else out


def stage_operand(x, threads: int = 1):
    """Fragments [mn/16][k/32][64][8] of a K-contiguous 16-bit operand: lane l
    of block (i, j) holds row 16i + l % 16, k = 32j + 8(l // 16) .. +7 ("cutlass
    入门", operand read of the matrix instruction; lane order of the AMD 16x16x32
    instruction)."""
    x = np.ascontiguousarray(x)
    if x.itemsize != 2 or x.ndim != 2:
        raise ValueError("2-D array of 16-bit elements")
    mn, k = x.shape
    out = np.empty((mn // 16, k // 32, 64, 8), dtype=x.dtype)
    if lib().oref_stage_operand(_ptr(x), _ptr(out), mn, k, threads) != 0:
        raise ValueError("oref_stage_operand rejected its arguments")
    return out
