"""Pins of the plain C oracle (oracle/c/oracle_ref.c), the one the CPU
baseline of the benchmark times.  Checked against the pages' worked example
and bit diagrams, against library routines (NumPy transposes and reshapes),
against brute force on tiny inputs, and for independence of the thread
split.  CPU only."""

import numpy as np
import pytest

import workloads as W
from conftest import read_kv, read_rows
from oracle import c_ref as C


def test_worked_example():
    g = read_kv("worked_example.txt")
    off = g["row"] * g["cols"] + g["col"]
    assert C.lib().oref_swizzle(off, g["B"], g["M"], g["S"]) == g["swizzled"]
    assert C.lib().oref_swizzle(off, g["B"], g["M"], 5) == g["swizzled_if_S5"]


def test_bit_diagrams():
    rng = np.random.default_rng(11)
    v = rng.integers(0, 2**31, size=1000).astype(np.int32)
    for name, B, M, S, zlo, ylo in read_rows("bit_diagrams.txt"):
        B, M, S, zlo, ylo = map(int, (B, M, S, zlo, ylo))
        yfield = ((1 << B) - 1) << ylo
        zfield = ((1 << B) - 1) << zlo
        got = C.swizzle_map(np.array([yfield, zfield, yfield | zfield], dtype=np.int32), B, M, S)
        assert list(got) == [yfield | zfield, zfield, yfield], name
        out = C.swizzle_map(v, B, M, S).view(np.uint32).astype(np.int64)
        vv = v.view(np.uint32).astype(np.int64)
        assert np.all((out ^ vv) & ~zfield == 0), name
        assert np.all(((out >> zlo) & ((1 << B) - 1)) == (((vv >> zlo) ^ (vv >> ylo)) & ((1 << B) - 1))), name


def test_map_permutes_and_inverts_itself():
    x = W.map_offsets(65536)
    for B, M, S in W.map_triples()[::7]:
        y = C.swizzle_map(x, B, M, S)
        assert np.array_equal(np.sort(y), x)
        assert np.array_equal(C.swizzle_map(y, B, M, S), x)


def test_map_rejects_out_of_range_triples():
    with pytest.raises(ValueError):
        C.swizzle_map(np.zeros(4, np.int32), 8, 12, 12)


@pytest.mark.parametrize("threads", [1, 3, 8])
@pytest.mark.parametrize("shape,dtype", [((96, 160), np.float32), ((130, 200), np.float16), ((1, 7), np.float32),
                                         ((77, 300), np.uint8),
                                         ((33, 1), np.uint16), ((0, 5), np.float32)])
def test_transpose_equals_library_transpose(shape, dtype, threads):
    rng = np.random.default_rng(3)
    a = rng.standard_normal(shape).astype(dtype)
    got = C.convert_layout(a, threads)
    assert got.shape == shape[::-1]
    assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(a.T).view(np.uint8))


@pytest.mark.parametrize("threads", [1, 5])
def test_batched_convert_equals_library_transpose(threads):
    a = W.bf16_tensor((5, 72, 136), seed=4)
    got = C.convert_layout(a, threads)
    assert np.array_equal(got, np.transpose(a, (0, 2, 1)))


def test_transpose_brute_force_tiny():
    a = np.arange(6, dtype=np.int32).reshape(2, 3)
    assert C.convert_layout(a).tolist() == [[0, 3], [1, 4], [2, 5]]


@pytest.mark.parametrize("threads", [1, 4])
def test_stage_operand_equals_reshape_form(threads):
    x = np.random.default_rng(5).integers(0, 2**16, size=(80, 96), dtype=np.uint16)
    got = C.stage_operand(x, threads)
    ref = x.reshape(5, 16, 3, 4, 8).transpose(0, 2, 3, 1, 4).reshape(5, 3, 64, 8)
    assert np.array_equal(got, ref)


def test_stage_operand_lane_contents():
    """Lane 37 of fragment (1, 2) holds row 16 + 5, k = 64 + 16 .. +7."""
    x = (np.arange(32 * 96, dtype=np.int64) % 65521).astype(np.uint16).reshape(32, 96)
    got = C.stage_operand(x)
    assert np.array_equal(got[1, 2, 37], x[21, 80:88])


def test_stage_operand_rejects_partial_fragments():
    with pytest.raises(ValueError):
        C.stage_operand(np.zeros((24, 32), np.uint16))


def test_negative_shift_matches_python_oracle_and_adjoint():
    import oracle as O

    rng = np.random.default_rng(12)
    x = rng.integers(0, 2 ** 31, size=2000).astype(np.int32)
    for B, M, S in [(3, 0, -3), (4, 3, -5), (2, 1, -1), (5, 2, -7)]:
        got = C.swizzle_map(x, B, M, S).view(np.uint32)
        assert np.array_equal(got, O.swizzle_signed(x.view(np.uint32), B, M, S))
