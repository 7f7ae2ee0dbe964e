"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here re-types the oracle's own formula: each test checks it against
a printed worked example, an independently stated form of the same map from
another page, a bit diagram, a closed form, an invariant or brute force.
"""

import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from conftest import read_kv, read_rows


# ---------------------------------------------------------------- swizzle map


def test_worked_example_offset_673():
    g = read_kv("worked_example.txt")
    off = g["row"] * g["cols"] + g["col"]
    assert off == g["offset"]
    out = O.swizzle(off, g["B"], g["M"], g["S"])
    assert out == g["swizzled"]
    assert divmod(out, g["cols"]) == (g["new_row"], g["new_col"])
    # the page's own (base, bits, shift) form, written independently
    assert O.swizzle_clear_set(off, g["M"], g["B"], g["S"]) == g["swizzled"]
    # reading note: a shift of 5 does not reproduce the page's result
    assert O.swizzle(off, g["B"], g["M"], 5) == g["swizzled_if_S5"]


@pytest.mark.parametrize(
    "rows,cols,params,coord_map",
    [
        # "CUDA 013 - Swizzle 的工作原理", section swizzle 映射案例: four coordinate maps
        (32, 32, (5, 0, 5), lambda y, x: (y, x ^ y)),
        (64, 32, (5, 0, 5), lambda y, x: (y, x ^ (y % 32))),
        (32, 64, (5, 0, 6), lambda y, x: (y, (x // 32) * 32 + ((x % 32) ^ y))),
        (32, 64, (5, 1, 5), lambda y, x: (y, (((x // 2) ^ y) * 2) + x % 2)),
    ],
)
def test_coordinate_forms_match_offset_form(rows, cols, params, coord_map):
    for y in range(rows):
        for x in range(cols):
            ny, nx = coord_map(y, x)
            assert O.swizzle(y * cols + x, *params) == ny * cols + nx


def test_bit_diagrams():
    for name, B, M, S, zlo, ylo in read_rows("bit_diagrams.txt"):
        B, M, S, zlo, ylo = map(int, (B, M, S, zlo, ylo))
        assert zlo == M and ylo == M + S, name
        yfield = ((1 << B) - 1) << ylo
        zfield = ((1 << B) - 1) << zlo
        # Y bits alone: Y stays, Z becomes Y (AA = ZZ xor YY with ZZ = 0)
        assert O.swizzle(yfield, B, M, S) == yfield | zfield, name
        # Z bits alone are untouched (YY = 0)
        assert O.swizzle(zfield, B, M, S) == zfield, name
        # Y and Z both set: Z cleared
        assert O.swizzle(yfield | zfield, B, M, S) == yfield, name
        rng = np.random.default_rng(7)
        for v in rng.integers(0, 2**31, size=200):
            v = int(v)
            out = O.swizzle(v, B, M, S)
            assert (out ^ v) & ~zfield == 0, name  # only Z may change
            ybits = (v >> ylo) & ((1 << B) - 1)
            assert ((out >> zlo) & ((1 << B) - 1)) == ((v >> zlo) & ((1 << B) - 1)) ^ ybits


def test_two_pages_forms_agree():
    """XOR form (handbook formula) against the clear/set form (offset-rule page)."""
    rng = np.random.default_rng(3)
    xs = [int(v) for v in rng.integers(0, 2**32, size=64)] + list(range(0, 4096, 7))
    for B, M, S in W.map_triples() + [(3, 0, 1), (4, 2, 2), (2, 5, 0)]:
        for x in xs:
            assert O.swizzle(x, B, M, S) == O.swizzle_clear_set(x, M, B, S)


def test_all_map_triples_bijective_and_involutive():
    x = W.map_offsets()
    for B, M, S in W.map_triples():
        y = O.swizzle_map(x, B, M, S)
        assert y.dtype == np.int32
        assert np.array_equal(np.sort(y), x), (B, M, S)  # permutation of 0..65535
        assert np.array_equal(O.swizzle_map(y, B, M, S), x), (B, M, S)  # S >= B


def test_overlapping_fields_bijective_not_involutive():
    x = np.arange(1 << 10, dtype=np.int32)
    y = O.swizzle_map(x, 3, 0, 1)
    assert np.array_equal(np.sort(y), x)
    assert not np.array_equal(O.swizzle_map(y, 3, 0, 1), x)


def test_blocks_are_permuted_in_place():
    """Only bits [M, M+B) change, so each aligned 2^(M+B) block maps onto itself."""
    x = W.map_offsets()
    for B, M, S in W.map_triples():
        y = O.swizzle_map(x, B, M, S).astype(np.int64)
        blk = 1 << (M + B)
        assert np.array_equal(y // blk, x // blk)
        assert np.array_equal(y % (1 << M), x % (1 << M))  # vectors of 2^M stay whole


def test_byte_units_equal_element_units():
    """The handbook counts M in bytes, the other pages in elements: with
    elements of 2^e bytes, Swizzle<B, M+e, S> on byte offsets equals
    Swizzle<B, M, S> on element offsets scaled by 2^e."""
    x = np.arange(1 << 14, dtype=np.int64)
    for e in range(4):
        for B, M, S in [(3, 3, 3), (3, 4, 3), (5, 0, 5), (2, 1, 4)]:
            lhs = O.swizzle(x << e, B, M + e, S).astype(np.int64)
            rhs = O.swizzle(x, B, M, S).astype(np.int64) << e
            assert np.array_equal(lhs, rhs)


def test_usage_example_int_32x128_rows_stay():
    """Offset-rule page, usage example 1: int[32][128] under (base 0, bits 5,
    shift 7) only permutes elements inside each row, and any column lands on
    32 different 4-byte banks."""
    rows, cols = 32, 128
    off = np.arange(rows * cols)
    new = O.swizzle(off, 5, 0, 7).astype(np.int64)
    assert np.array_equal(new // cols, off // cols)
    grid = new.reshape(rows, cols)
    for x in range(cols):
        assert len(set((grid[:, x] % 32).tolist())) == 32


def test_usage_example_int_32x8_rows_grouped_by_four():
    """Usage example 4: int[32][8] with bits 5 and shift 5 treats four rows as
    one 32-wide bank row: elements stay inside their group of four rows and a
    column read over all 32 rows hits 32 different banks.

    Reading: the page adds that elements then move between rows; at 32 rows
    the two top source bits (offset bits 8 and 9) are zero, so each element
    keeps its row here.  Rows do move once the matrix has 128 rows or more."""
    rows, cols = 32, 8
    off = np.arange(rows * cols)
    new = O.swizzle(off, 5, 0, 5).astype(np.int64)
    assert np.array_equal((new // cols) // 4, (off // cols) // 4)
    assert np.array_equal(new // cols, off // cols)
    grid = new.reshape(rows, cols)
    for x in range(cols):
        assert len(set((grid[:, x] % 32).tolist())) == 32
    taller = np.arange(128 * cols)
    moved = O.swizzle(taller, 5, 0, 5).astype(np.int64)
    assert np.array_equal((moved // cols) // 4, (taller // cols) // 4)
    assert not np.array_equal(moved // cols, taller // cols)


# ------------------------------------------------------------ tile addresses


def test_tile_offsets_are_one_to_one():
    for layout, params, pad in [("swizzle", (5, 0, 5), 0), ("pad", None, 1), ("plain", None, 0)]:
        r, c = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
        off = O.tile_offset(r.ravel(), c.ravel(), 32, layout, params, pad)
        assert len(set(off.tolist())) == 32 * 32
    assert O.tile_offset(1, 0, 32, "pad", pad=1) == 33


# ------------------------------------------------------- conflict counter


def _col_read(rows, width_words, col, stride):
    return [l * stride * 4 + col * 4 for l in range(rows)]


def test_conflicts_column_of_8x32_fp32():
    """Handbook, typical scenario: column 0 of an 8x32 fp32 tile puts every
    lane on bank 0 (8-way); a row read is conflict-free."""
    nv = O.nvidia_model()
    addrs = [r * 32 * 4 for r in range(8)] + [None] * 24
    cyc, worst, _ = O.conflict_report(addrs, 4, nv)
    assert worst == 8 and cyc == 7
    row = [c * 4 for c in range(32)]
    assert O.conflict_report(row, 4, nv)[1] == 1


def test_conflicts_32x32_column_pad_and_xor():
    nv = O.nvidia_model()
    col = [r * 32 * 4 for r in range(32)]
    assert O.conflict_report(col, 4, nv)[1] == 32
    padded = [r * 33 * 4 for r in range(32)]  # the 32x33 array
    assert O.conflict_report(padded, 4, nv)[1] == 1
    for x in range(32):
        xor = [(r * 32 + (x ^ r)) * 4 for r in range(32)]  # mapping (y, x^y)
        assert O.conflict_report(xor, 4, nv)[1] == 1


def test_conflicts_broadcast_and_subword():
    nv = O.nvidia_model()
    assert O.conflict_report([64] * 32, 4, nv)[1] == 1  # one address: broadcast
    halves = [(l // 2) * 4 + (l % 2) * 2 for l in range(32)]  # two f16 per word
    assert O.conflict_report(halves, 2, nv)[1] == 1
    same_bank = [(l % 2) * 128 for l in range(32)]  # two words of bank 0
    assert O.conflict_report(same_bank, 4, nv)[1] == 2


@pytest.mark.parametrize("stride", range(1, 70))
def test_conflicts_stride_closed_form(stride):
    """32 lanes reading word l*stride of 32 one-word banks: the degree is
    gcd(stride, 32) (the lanes fall into 32/gcd distinct banks, evenly)."""
    nv = O.nvidia_model()
    addrs = [l * stride * 4 for l in range(32)]
    assert O.conflict_report(addrs, 4, nv)[1] == math.gcd(stride, 32)


def test_wide_access_minimum_phases_are_not_conflicts():
    """"NVIDIA CuTe Swizzle": a 16x16 f16 ldmatrix.x4 needs four phases; that
    is not a conflict.  32 lanes x 16 bytes over contiguous memory."""
    nv = O.nvidia_model()
    cyc, worst, degrees = O.conflict_report([l * 16 for l in range(32)], 16, nv)
    assert cyc == 0 and worst == 1 and degrees == [1, 1, 1, 1]


def test_model_64_banks_changes_the_plain_column_degree():
    """The same 32x32 fp32 column read is 16-way under 64 banks x 4 bytes with
    64-lane phases (rows of 128 bytes alternate between the two bank halves)."""
    h64 = O.BankModel(64, 4, 64)
    col2 = [(l % 32) * 128 + (l // 32) * 4 for l in range(64)]
    assert O.conflict_report(col2, 4, h64)[1] == 16


# -------------------------------------------------------------- the chooser


def _column_read_instrs(esz, vec_bytes, rows, cols, n_lanes):
    ve = vec_bytes // esz
    instrs = []
    for c in range(0, cols, ve):
        for r0 in range(0, rows, n_lanes):
            coords = [(r0 + l, c) if r0 + l < rows else None for l in range(n_lanes)]
            instrs.append((coords, vec_bytes))
    return instrs


def _row_write_instrs(esz, vec_bytes, rows, cols, n_lanes):
    ve = vec_bytes // esz
    nvec = rows * cols // ve
    instrs = []
    for base in range(0, nvec, n_lanes):
        coords = []
        for l in range(n_lanes):
            v = base + l
            coords.append(divmod(v * ve, cols) if v < nvec else None)
        instrs.append((coords, vec_bytes))
    return instrs


def test_chooser_reproduces_the_pages_choices():
    nv = O.nvidia_model()
    for name, esz, vb, tr, tc, lanes, B, M, S in read_rows("usage_examples.txt"):
        esz, vb, tr, tc, lanes, B, M, S = map(int, (esz, vb, tr, tc, lanes, B, M, S))
        wr = _row_write_instrs(esz, vb, tr, tc, 32)
        rd = _column_read_instrs(esz, vb, tr, tc, 32)
        (b, m, s), cyc = O.choose(esz, vb, tr, tc, wr, rd, nv)
        assert cyc == 0, name
        # same map over the tile as the page's triple (the int[32][8] example
        # names a 5-bit field whose top two source bits lie outside the tile)
        x = np.arange(tr * tc)
        assert np.array_equal(O.swizzle(x, b, m, s), O.swizzle(x, B, M, S)), (name, (b, m, s))
        assert pytest.approx(1 << m) == vb // esz


def test_chooser_minimum_over_search_space():
    """Brute force: nothing in the (B,M,S) space beats the chooser's cycles."""
    h64 = O.BankModel(64, 4, 64)
    esz, vb, tr, tc = 2, 16, 64, 64
    wr = _row_write_instrs(esz, vb, tr, tc, 64)
    rd = _column_read_instrs(esz, vb, tr, tc, 64)
    (b, m, s), cyc = O.choose(esz, vb, tr, tc, wr, rd, h64)
    best = min(
        O.pattern_cycles(wr, tc, esz, "swizzle", h64, (B, 3, S))[0]
        + O.pattern_cycles(rd, tc, esz, "swizzle", h64, (B, 3, S))[0]
        for B in range(0, 5)
        for S in range(0, 9)
        if 3 + B + S <= 12
    )
    assert cyc == best


# --------------------------------------------------------- data movement


def test_transpose_adjoint_identity():
    """<A^T x, y> = <x, A y> for every x, y: checked with a library matmul on
    the original matrix, so a wrong index or a copy instead of a transpose fails."""
    rng = np.random.default_rng(0)
    for rows, cols in [(1, 1), (1, 7), (5, 1), (33, 65), (64, 32)]:
        a = rng.standard_normal((rows, cols))
        at = O.transpose(a)
        assert at.shape == (cols, rows)
        x = rng.standard_normal(rows)
        y = rng.standard_normal(cols)
        assert np.isclose((at @ x) @ y, x @ (a @ y))
        assert np.array_equal(O.transpose(at), a)
    sym = rng.standard_normal((9, 9))
    sym = sym + sym.T
    assert np.array_equal(O.transpose(sym), sym)


def test_transpose_is_bitwise():
    bits = W.fp32_matrix(17, 40, seed=5)
    t = O.transpose(bits)
    assert t.dtype == np.uint32
    assert t[3, 11] == bits[11, 3] and t[39, 16] == bits[16, 39]


def test_convert_layout_per_batch():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((3, 6, 10))
    out = O.convert_layout(a)
    for b in range(3):
        x = rng.standard_normal(6)
        y = rng.standard_normal(10)
        assert np.isclose((out[b] @ x) @ y, x @ (a[b] @ y))
    assert O.convert_layout(np.zeros((0, 4, 5))).shape == (0, 5, 4)


def test_stage_operand_loops_and_reshape_forms():
    rng = np.random.default_rng(2)
    x = rng.integers(0, 2**16, size=(48, 96), dtype=np.uint16)
    frag = O.stage_operand(x)
    assert np.array_equal(frag, O.stage_operand_loops(x))
    alt = x.reshape(3, 16, 3, 4, 8).transpose(0, 2, 3, 1, 4).reshape(3, 3, 64, 8)
    assert np.array_equal(frag, alt)


def test_stage_operand_fragments_multiply_like_the_operands():
    """Fragments of A and of B^T, combined lane group by lane group the way a
    16x16x32 product consumes them, give A_blk @ B_blk (library matmul)."""
    rng = np.random.default_rng(4)
    a = rng.standard_normal((32, 64))
    bt = rng.standard_normal((48, 64))
    fa, fb = O.stage_operand(a), O.stage_operand(bt)
    for i in range(2):
        for n in range(3):
            c = np.zeros((16, 16))
            for j in range(2):
                for g in range(4):
                    c += fa[i, j, 16 * g:16 * g + 16, :] @ fb[n, j, 16 * g:16 * g + 16, :].T
            ref = a[16 * i:16 * i + 16] @ bt[16 * n:16 * n + 16].T
            assert np.allclose(c, ref)


def test_stage_operand_rejects_partial_fragments():
    with pytest.raises(ValueError):
        O.stage_operand(np.zeros((17, 32), dtype=np.uint16))


# ------------------------------------------------- consumer of the fragments


def test_bf16_decode_known_values():
    # bf16 patterns of 1.0, -2.0, 0.5 and the smallest normal
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0080], dtype=np.uint16)
    assert list(O.bf16_to_f64(bits)) == [1.0, -2.0, 0.5, 2.0 ** -126]


def _bf16_bits_of_ints(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_gemm_matches_brute_force_integer_products():
    """Small integers are exact in bf16; the product is checked against a
    pure-Python triple loop, with A and B of different shapes so a swapped
    or untransposed operand cannot pass."""
    rng = np.random.default_rng(8)
    a = rng.integers(-3, 4, size=(5, 7))
    bt = rng.integers(-3, 4, size=(3, 7))
    got = O.gemm_bf16(_bf16_bits_of_ints(a), _bf16_bits_of_ints(bt))
    assert got.shape == (5, 3)
    for i in range(5):
        for j in range(3):
            assert got[i, j] == sum(int(a[i, t]) * int(bt[j, t]) for t in range(7))


def test_gemm_through_fragments_equals_gemm():
    """Multiplying the oracle's fragments block by block, lane group by lane
    group, reproduces the oracle's product (the fragment layout is what the
    consumer relies on)."""
    rng = np.random.default_rng(9)
    a = _bf16_bits_of_ints(rng.integers(-2, 3, size=(32, 64)))
    bt = _bf16_bits_of_ints(rng.integers(-2, 3, size=(48, 64)))
    fa, fb = O.stage_operand(a), O.stage_operand(bt)
    ref = O.gemm_bf16(a, bt)
    for i in range(2):
        for n in range(3):
            acc = np.zeros((16, 16))
            for j in range(2):
                for g in range(4):
                    acc += O.bf16_to_f64(fa[i, j, 16 * g:16 * g + 16]) @ O.bf16_to_f64(fb[n, j, 16 * g:16 * g + 16]).T
            assert np.array_equal(acc, ref[16 * i:16 * i + 16, 16 * n:16 * n + 16])


def test_gemm_error_bound_covers_fp32_accumulation():
    """The bound holds for an actual fp32 chunked accumulation of random
    bf16 data (computed here with float32 NumPy arithmetic)."""
    rng = np.random.default_rng(10)
    a32 = rng.standard_normal((8, 256)).astype(np.float32)
    b32 = rng.standard_normal((6, 256)).astype(np.float32)
    a = (a32.view(np.uint32) >> 16).astype(np.uint16)
    bt = (b32.view(np.uint32) >> 16).astype(np.uint16)
    av, bv = O.bf16_to_f64(a).astype(np.float32), O.bf16_to_f64(bt).astype(np.float32)
    acc = np.zeros((8, 6), dtype=np.float32)
    for c0 in range(0, 256, 32):
        acc = acc + (av[:, c0:c0 + 32] @ bv[:, c0:c0 + 32].T).astype(np.float32)
    err = np.abs(acc.astype(np.float64) - O.gemm_bf16(a, bt))
    assert np.all(err <= O.gemm_error_bound(a, bt))


def _bf16(vals):
    """bf16 bits of values that bf16 holds exactly."""
    return (np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _adversarial_chunks(k=4096):
    """One row of A and of B^T whose 32-wide chunk sums are exact in fp32 and
    whose fp32 accumulation rounds the same way at every step: chunk 0 sums
    to 2^24 (one fp32 step there is 2), every later chunk to 1 + 2^-8, so each
    add lands 1 + 2^-8 above an even number and rounds up by 1 - 2^-8."""
    a, b = np.zeros(k, np.float32), np.zeros(k, np.float32)
    a[0] = b[0] = 2.0 ** 12
    for c0 in range(32, k, 32):
        a[c0] = b[c0] = 1.0
        a[c0 + 1] = b[c0 + 1] = 2.0 ** -4
    return _bf16(a[None, :]), _bf16(b[None, :])


def _fp32_chunked(a_bits, bt_bits, chunks=None):
    """fp32 accumulation of 32-wide chunk sums in k order (the matrix
    instruction's k step), optionally over a subset of the chunks."""
    av, bv = O.bf16_to_f64(a_bits).astype(np.float32), O.bf16_to_f64(bt_bits).astype(np.float32)
    k = av.shape[1]
    acc = np.zeros((av.shape[0], bv.shape[0]), dtype=np.float32)
    for j in (range(k // 32) if chunks is None else chunks):
        acc = acc + (av[:, 32 * j:32 * j + 32] @ bv[:, 32 * j:32 * j + 32].T).astype(np.float32)
    return acc.astype(np.float64)


def test_gemm_error_bound_is_reached_within_a_small_factor():
    """From above: on inputs whose fp32 rounding errors all point one way the
    observed error comes within 1.3x of the bound (126.5 against 160 at
    k = 4096), so the bound is not loose by a dropped 2^-24, a step count of
    k instead of k/32, or any other factor of 1.5 or more."""
    a, bt = _adversarial_chunks(4096)
    exact = O.gemm_bf16(a, bt)
    assert exact[0, 0] == 2.0 ** 24 + 127 * (1 + 2.0 ** -8)  # the chunk sums are what the construction says
    err = abs(_fp32_chunked(a, bt)[0, 0] - exact[0, 0])
    bound = O.gemm_error_bound(a, bt)[0, 0]
    assert err <= bound <= 1.5 * err
    assert 126 < err < 127


def test_loosened_bounds_fail_the_tightness_check():
    """The check above tells a plausible mistake in the bound apart: the same
    bound without its 2^-24 factor, or with k steps instead of k/32, is more
    than 1.5x the adversarial error."""
    a, bt = _adversarial_chunks(4096)
    err = abs(_fp32_chunked(a, bt)[0, 0] - O.gemm_bf16(a, bt)[0, 0])
    bound = O.gemm_error_bound(a, bt)[0, 0]
    k = 4096
    for loose in (bound * 2.0 ** 24, bound * (k + 32) / (k // 32 + 32)):
        assert loose > 1.5 * err


def test_a_dropped_chunk_exceeds_the_gemm_error_bound():
    """The bound is small enough for the GPU GEMM tests to see a lost k chunk:
    on operands drawn like the staging workload (normal(0, 0.02), k = 4096),
    leaving one 32-wide chunk out of the fp32 accumulation moves nearly every
    element by more than the bound."""
    rng = np.random.default_rng(11)
    a = _bf16(rng.standard_normal((16, 4096)).astype(np.float32) * np.float32(0.02))
    bt = _bf16(rng.standard_normal((16, 4096)).astype(np.float32) * np.float32(0.02))
    exact, bound = O.gemm_bf16(a, bt), O.gemm_error_bound(a, bt)
    assert np.all(np.abs(_fp32_chunked(a, bt) - exact) <= bound)
    dropped = _fp32_chunked(a, bt, [j for j in range(128) if j != 77])
    assert np.mean(np.abs(dropped - exact) > bound) > 0.9


# ------------------------------------------------------ negative shifts


def _parity(v):
    return bin(int(v)).count("1") & 1


@pytest.mark.parametrize("B,M,S", [(3, 0, 3), (3, 3, 4), (2, 5, 7), (5, 0, 5), (4, 2, 1), (1, 9, 11)])
def test_negative_shift_is_the_transpose_of_the_positive_one(B, M, S):
    """Over GF(2) the swizzle is I + N, where N copies the source field onto
    the target; reversing the shift swaps source and target, i.e. replaces N
    by its transpose.  So <sw(x; -S), y> = <x, sw(y; S)> for the bitwise dot
    product -- a fact about the maps, not a restatement of the formula."""
    rng = np.random.default_rng(B * 100 + M * 10 + S)
    for x, y in rng.integers(0, 2 ** 31, size=(300, 2)):
        lhs = _parity(O.swizzle_signed(int(x), B, M, -S) & int(y))
        rhs = _parity(int(x) & O.swizzle_signed(int(y), B, M, S))
        assert lhs == rhs


def test_negative_shift_moves_the_low_field_left():
    """The SShift comment: a negative shift moves the YYY mask left.  With
    only the low field (at M) set, the result also carries it |S| higher."""
    for B, M, S in [(3, 4, -6), (2, 3, -11), (5, 0, -5)]:
        low = ((1 << B) - 1) << M
        assert O.swizzle_signed(low, B, M, S) == low | (low << -S)
        high = low << -S
        assert O.swizzle_signed(high, B, M, S) == high  # the target alone is left alone


def test_signed_form_agrees_with_the_positive_form():
    rng = np.random.default_rng(3)
    x = rng.integers(0, 2 ** 31, size=500)
    for B, M, S in [(3, 3, 3), (5, 0, 6), (2, 4, 1)]:
        assert np.array_equal(O.swizzle_signed(x, B, M, S), O.swizzle(x, B, M, S))


@pytest.mark.parametrize("B,M,S", [(3, 0, -3), (4, 3, -5), (2, 1, -1), (5, 0, -2)])
def test_negative_shift_bijective_and_involutive_when_fields_apart(B, M, S):
    x = np.arange(1 << 14, dtype=np.int64)
    y = O.swizzle_signed(x, B, M, S).astype(np.int64)
    assert np.array_equal(np.sort(y), x)  # one-to-one
    if -S >= B:
        assert np.array_equal(O.swizzle_signed(y, B, M, S).astype(np.int64), x)


# ---------------------------------------------- folding into a plain layout


def test_fold_collision_truth_table():
    """[Intro] swizzle 融入 layout 优化: for one source/target bit pair, the
    collision bit is set only when both are active (the page's table)."""
    B, M, S = 1, 2, 3  # target bit 2, source bit 5
    for a_z in (0, 1):
        for a_y in (0, 1):
            active = (a_z << 2) | (a_y << 5)
            assert O.fold_collision(active, B, M, S) == (a_z & a_y) << 2


def _subsets(mask):
    bits = [b for b in range(32) if (mask >> b) & 1]
    for r in range(1 << len(bits)):
        yield sum(1 << bits[i] for i in range(len(bits)) if (r >> i) & 1)


def test_fold_matches_brute_force_additivity():
    """Brute force over every offset of small slices: the swizzle is a plain
    (additive) layout on the slice exactly when there is no collision, and
    then the folded strides reproduce every offset."""
    rng = np.random.default_rng(21)
    seen = {True: 0, False: 0}
    for _ in range(300):
        B = int(rng.integers(1, 4))
        M = int(rng.integers(0, 4))
        S = int(rng.choice([-1, 1])) * int(rng.integers(1, 6))
        bits = rng.choice(12, size=int(rng.integers(1, 7)), replace=False)
        active = sum(1 << int(b) for b in bits)
        base = int(rng.integers(0, 1 << 12)) & ~active
        coll = O.fold_collision(active, B, M, S)
        sb, strides = O.fold_strides(base, active, B, M, S)
        additive = all(int(O.swizzle_signed(base | x, B, M, S)) ==
                       sb + sum(strides[b] for b in strides if (x >> b) & 1) for x in _subsets(active))
        assert additive == (coll == 0), (B, M, S, active, base)
        seen[coll == 0] += 1
    assert seen[True] > 20 and seen[False] > 20


# ------------------------------------------------------ bf16 rounding


def test_bf16_rounding_matches_the_library_conversion():
    """The oracle's nearest-even rounding to bf16 against torch's fp32 ->
    bfloat16 conversion (round to nearest even) on values of every size,
    exact ties included."""
    import torch

    rng = np.random.default_rng(31)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        # exact ties: an upper half with the low 16 bits 0x8000
        ((rng.integers(0x0080, 0x7F00, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max, -np.finfo(np.float32).max,
                  np.finfo(np.float32).tiny, 1e-45], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), ref)


def test_bf16_rounding_ties_go_to_even_and_nan_stays_nan():
    one = np.float32(1.0)
    half_ulp, ulp = np.float32(2.0 ** -8), np.float32(2.0 ** -7)
    got = O.f32_to_bf16_bits(np.array([one, one + half_ulp, one + ulp + half_ulp, -(one + half_ulp)],
                                      dtype=np.float32))
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0xBF80]
    assert O.f32_to_bf16_bits(np.array([np.finfo(np.float32).max], dtype=np.float32))[0] == 0x7F80  # to infinity
    nan = O.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0
    # the bf16 values themselves are fixed points
    b = np.arange(0, 0x7F80, 7, dtype=np.uint32)
    assert np.array_equal(O.f32_to_bf16_bits((b << 16).view(np.float32)), b.astype(np.uint16))
