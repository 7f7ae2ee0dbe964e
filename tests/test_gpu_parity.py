"""Bit-exact parity of the HIP path against the CPU oracle (needs a GPU).

Every call goes through the C ABI (libswz.so) via the thin ctypes binding.
Inputs come from the seeded generators in ``workloads``; expected values from
``oracle`` only.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W

import torch  # noqa: E402  (hard imports: a GPU run without them fails, never skips)

import tiled_movement_amd as T  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SIGNED = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32, np.dtype(np.int32): np.int32,
          np.dtype(np.uint8): np.uint8}


def to_dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(SIGNED[a.dtype])).to(DEV)


def from_dev(t, like):
    return t.cpu().numpy().view(like.dtype)


def announce(*what):
    print("case:", *what, flush=True)


# ------------------------------------------------------------------ map


def test_map_every_triple_full_range():
    x = W.map_offsets()
    xin = to_dev(x)
    out = torch.empty_like(xin)
    for B, M, S in W.map_triples():
        T.swz_map(xin, out, x.size, (B, M, S))
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(out, x), O.swizzle_map(x, B, M, S)), (B, M, S)


def test_map_worked_example_and_edges():
    announce("map edges")
    x = W.map_offsets(4099)
    xin = to_dev(x)
    out = torch.empty_like(xin)
    T.swz_map(xin, out, x.size, (5, 0, 6))
    torch.cuda.synchronize()
    got = from_dev(out, x)
    assert got[673] == 683
    assert np.array_equal(got, O.swizzle_map(x, 5, 0, 6))
    # misaligned (4-byte offset) pointers take the scalar path; odd length
    T.swz_map(xin[1:], out[1:], x.size - 1, (3, 2, 4))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out, x)[1:], O.swizzle_map(x[1:], 3, 2, 4))
    # in place
    y = xin.clone()
    T.swz_map(y, y, x.size, (4, 1, 5))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(y, x), O.swizzle_map(x, 4, 1, 5))
    # identity and the whole 32-bit range of bit patterns
    rng = np.random.default_rng(11)
    z = rng.integers(-(2**31), 2**31, size=1000, dtype=np.int64).astype(np.int32)
    zin = to_dev(z)
    zout = torch.empty_like(zin)
    for p in [(0, 0, 0), (5, 4, 7), (8, 16, 8), (1, 30, 1)]:
        T.swz_map(zin, zout, z.size, p)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(zout, z), O.swizzle_map(z, *p)), p
    T.swz_map(zin, zout, 0, (5, 0, 5))  # n = 0 is a no-op


def test_map_negative_shifts():
    announce("map negative shifts")
    rng = np.random.default_rng(13)
    z = rng.integers(-(2**31), 2**31, size=4099, dtype=np.int64).astype(np.int32)
    zin = to_dev(z)
    zout = torch.empty_like(zin)
    for p in [(3, 0, -3), (5, 0, -5), (4, 3, -7), (2, 1, -1), (8, 8, -16), (1, 0, -31)]:
        T.swz_map(zin, zout, z.size, p)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(zout, z), O.swizzle_map(z, *p)), p


def test_map_batch_every_triple_one_launch():
    """The map's workload in one call: 0..65535 under all 125 triples."""
    announce("map batch 125")
    x = W.map_offsets()
    triples = W.map_triples()
    xin = to_dev(x)
    out = torch.empty((len(triples), x.size), dtype=xin.dtype, device=DEV)
    T.swz_map_batch(xin, out, x.size, triples)
    torch.cuda.synchronize()
    got = from_dev(out, x).reshape(len(triples), x.size)
    for j, (B, M, S) in enumerate(triples):
        assert np.array_equal(got[j], O.swizzle_map(x, B, M, S)), (B, M, S)
    assert got[triples.index((5, 0, 6))][673] == 683


def test_map_batch_chunks_odd_lengths_and_signs():
    """More triples than one launch takes (300: three launches), either sign
    of S, odd n (scalar path) and a misaligned input, over 32-bit patterns."""
    rng = np.random.default_rng(17)
    triples = []
    while len(triples) < 300:
        B, M = int(rng.integers(0, 9)), int(rng.integers(0, 12))
        S = int(rng.integers(-12, 13))
        if B + M + abs(S) <= 32:
            triples.append((B, M, S))
    z = rng.integers(-(2**31), 2**31, size=1001, dtype=np.int64).astype(np.int32)
    zin = to_dev(z)
    for n, src in ((z.size, zin), (z.size - 1, zin[1:])):
        announce("map batch chunks", n)
        out = torch.empty((len(triples), n), dtype=zin.dtype, device=DEV)
        T.swz_map_batch(src, out, n, triples)
        torch.cuda.synchronize()
        got = from_dev(out, z).reshape(len(triples), n)
        ref = z[z.size - n:]
        for j, p in enumerate(triples):
            assert np.array_equal(got[j], O.swizzle_map(ref, *p)), p
    T.swz_map_batch(zin, zin, 0, triples)  # n = 0 is a no-op


# ----------------------------------------------------------- transposes

KINDS = [
    (T.READ_SCALAR_COL, 4, 32, 32, W.fp32_matrix),
    (T.READ_B64_4X4, 2, 64, 64, W.fp16_matrix),
    (T.READ_B128_8X8, 2, 64, 128, lambda r, c, seed: W.bf16_tensor((r, c), seed=seed)),
    (T.READ_B64_TR16, 2, 64, 64, W.fp16_matrix),
    (T.READ_B64_TR8, 1, 128, 128, W.u8_matrix),
]
LAYOUTS = ["swizzle", "pad", "plain"]


def shapes_for(tr, tc):
    return [
        (3 * tr, 2 * tc),  # whole tiles
        (2 * tr + 5, 3 * tc + 3),  # ragged tails in both directions
        (3 * tr + 7, 2 * tc + 5),  # an odd count of whole tile rows, then a ragged one
        (tr - 1, tc + 1),
        (1, 1),
        (1, 5 * tc + 7),
        (4 * tr + 3, 1),
        (0, 7),
        (7, 0),
    ]


def check_transpose(a, esz, layout, kind, params=None):
    rows, cols = a.shape
    src = to_dev(a)
    dst = torch.empty((cols, rows), dtype=src.dtype, device=DEV)
    T.swz_transpose(src, dst, rows, cols, esz, layout, kind, params)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dst, a), O.transpose(a)), (a.shape, layout, kind, params)


@pytest.mark.parametrize("kind,esz,tr,tc,gen", KINDS)
@pytest.mark.parametrize("layout", LAYOUTS)
def test_transpose_shapes(kind, esz, tr, tc, gen, layout):
    for seed, (rows, cols) in enumerate(shapes_for(tr, tc)):
        announce("transpose", kind, layout, rows, cols)
        check_transpose(gen(rows, cols, seed=seed), esz, layout, kind)


@pytest.mark.parametrize("kind,esz,tr,tc,gen", KINDS)
def test_transpose_unaligned_pointers(kind, esz, tr, tc, gen):
    """Sources and destinations one element off a 16-byte boundary."""
    rows, cols = 2 * tr + 8, 2 * tc + 8
    a = gen(rows, cols, seed=3)
    flat = to_dev(a.reshape(-1))
    buf = torch.empty(a.size + 1, dtype=flat.dtype, device=DEV)
    buf[1:] = flat
    out = torch.empty(a.size + 1, dtype=flat.dtype, device=DEV)
    announce("unaligned", kind)
    T.swz_transpose(buf[1:], out[1:], rows, cols, esz, "swizzle", kind)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out[1:], a).reshape(cols, rows), O.transpose(a))


@pytest.mark.parametrize("kind,esz,tr,tc,gen", KINDS)
def test_transpose_any_valid_swizzle(kind, esz, tr, tc, gen):
    """The swizzle only moves data inside LDS: every admissible (B, M, S)
    gives the same bits out."""
    rows, cols = 2 * tr + 3, 2 * tc + 5
    a = gen(rows, cols, seed=4)
    m_min = {4: 0, 2: 3, 1: 3}[esz]
    log_tile = (tr * tc).bit_length() - 1
    rng = np.random.default_rng(kind)
    triples = [(B, M, S) for B in range(1, 6) for M in range(m_min, 6) for S in range(1, 9)
               if M + B <= log_tile]
    for idx in rng.choice(len(triples), size=min(12, len(triples)), replace=False):
        announce("params", kind, triples[idx])
        check_transpose(a, esz, "swizzle", kind, triples[idx])


@pytest.mark.parametrize("kind,esz,tr,tc,gen", KINDS)
def test_transpose_negative_shifts(kind, esz, tr, tc, gen):
    """Negative shifts XOR a low field into a higher one; the data still only
    moves inside LDS, so the transpose is unchanged."""
    q = 16 // esz  # ragged by one 16-byte run, so the direct layout's pitch rule holds
    rows, cols = 2 * tr + q, 2 * tc + q
    a = gen(rows, cols, seed=24)
    m0 = 0 if esz == 4 else 3  # 2-byte: 16-byte vectors; 1-byte: 8-byte runs
    log_tile = (tr * tc).bit_length() - 1
    for B, M, S in [(3, m0, -3), (2, m0, -5), (3, m0 + 1, -4), (1, m0, -1)]:
        if M - S + B > log_tile:
            continue
        for layout in ("swizzle", "direct") if -S >= B else ("swizzle",):
            announce("negative shift", kind, layout, (B, M, S))
            check_transpose(a, esz, layout, kind, (B, M, S))


def test_convert_layout_batches():
    cases = [
        (T.READ_B128_8X8, 2, W.bf16_tensor((3, 200, 128), seed=5)),
        (T.READ_B128_8X8, 2, W.bf16_tensor((2, 64, 100), seed=6)),  # ragged rows of 100
        (T.READ_B64_4X4, 2, W.bf16_tensor((2, 70, 130), seed=7)),
        (T.READ_B64_TR16, 2, W.bf16_tensor((2, 70, 130), seed=10)),
        (T.READ_B64_TR8, 1, W.u8_matrix(3 * 130, 200, seed=11).reshape(3, 130, 200)),
        (T.READ_SCALAR_COL, 4, W.fp32_matrix(3 * 40, 50, seed=8).reshape(3, 40, 50)),
        # stacked whole-tile blocks per batch entry: 2 x 2 fp32 tiles with a whole tile row and
        # a whole tile column left over, and two 16-bit tiles down the rows with one left over
        (T.READ_SCALAR_COL, 4, W.fp32_matrix(2 * 100, 100, seed=20).reshape(2, 100, 100)),
        (T.READ_SCALAR_COL, 4, W.fp32_matrix(3 * 96, 136, seed=21).reshape(3, 96, 136)),
        (T.READ_B64_4X4, 2, W.bf16_tensor((3, 200, 136), seed=22)),
        (T.READ_B64_TR16, 2, W.bf16_tensor((2, 192, 264), seed=23)),
    ]
    for kind, esz, a in cases:
        for layout in LAYOUTS:
            announce("convert", kind, layout, a.shape)
            b, r, c = a.shape
            src = to_dev(a)
            dst = torch.empty((b, c, r), dtype=src.dtype, device=DEV)
            T.swz_convert_layout(src, dst, b, r, c, esz, layout, kind)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(dst, a), O.convert_layout(a))


def test_auto_read_kind():
    for shape in [(4, 96, 128), (2, 100, 300)]:  # narrow rows -> 8x8 reads; wide -> transpose reads
        a = W.bf16_tensor(shape, seed=9)
        b, r, c = shape
        announce("auto", shape, T.swz_plan(0, r, c, 2)["read_kind"])
        src = to_dev(a)
        dst = torch.empty((b, c, r), dtype=src.dtype, device=DEV)
        T.swz_convert_layout(src, dst, b, r, c, 2)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst, a), O.convert_layout(a))


# ------------------------------- narrow rows (whole-row tiles, 1 to 64 bytes)
GEN = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}
NARROW_KINDS = ([(k, 4, c) for k, c in zip((T.READ_NARROW1, T.READ_NARROW2, T.READ_NARROW4, T.READ_NARROW8,
                                             T.READ_NARROW16), (1, 2, 4, 8, 16))] +
                [(k, 2, c) for k, c in zip((T.READ_HNARROW1, T.READ_HNARROW2, T.READ_HNARROW4, T.READ_HNARROW8,
                                             T.READ_HNARROW16, T.READ_HNARROW32), (1, 2, 4, 8, 16, 32))] +
                [(k, 1, c) for k, c in zip((T.READ_BNARROW1, T.READ_BNARROW2, T.READ_BNARROW4, T.READ_BNARROW8,
                                             T.READ_BNARROW16, T.READ_BNARROW32, T.READ_BNARROW64),
                                            (1, 2, 4, 8, 16, 32, 64))])


@pytest.mark.parametrize("kind,esz,c", NARROW_KINDS)
@pytest.mark.parametrize("layout", LAYOUTS + ["direct"])
def test_narrow_rows(kind, esz, c, layout):
    """Whole-row tiles, the swizzle spanning several rows: whole tiles,
    ragged last tiles (on and off a 16-byte output pitch), fewer rows than
    one tile, empty."""
    tr = T.swz_plan(0, 4096, c, esz, "swizzle", kind)["tile"][0]
    if layout == "pad" and c * esz < 4:  # rows under one 4-byte LDS store get no pad
        with pytest.raises(T.SwzError):
            check_transpose(GEN[esz](tr, c, seed=0), esz, layout, kind)
        return
    for seed, rows in enumerate([3 * tr, 2 * tr + 16, 2 * tr + 4, 2 * tr + 3, tr - 16, tr - 4, 5, 1, 0]):
        if layout == "direct" and (rows * esz) % 16:
            continue  # the direct fill needs a 16-byte output pitch
        announce("narrow", kind, layout, rows, c)
        check_transpose(GEN[esz](rows, c, seed=seed), esz, layout, kind)


@pytest.mark.parametrize("kind,esz,c", NARROW_KINDS)
def test_narrow_auto_unaligned_and_batched(kind, esz, c):
    rows = 3 * T.swz_plan(0, 4096, c, esz, "swizzle", kind)["tile"][0] + 9
    # output rows of 9 elements past whole tiles are no multiple of 16 bytes: AUTO takes flat rows for
    # every fp32 width, 2-byte widths of 8 to 32 and bytes x 64 (the explicit kind is tested below)
    to_rows = esz == 4 or (esz == 2 and c >= 8) or (esz == 1 and c == 64)
    assert T.swz_plan(0, rows, c, esz)["read_kind"] == (T.READ_ROWS if to_rows else kind)
    a = GEN[esz](rows, c, seed=c)
    announce("narrow auto", esz, c)
    check_transpose(a, esz, "swizzle", T.READ_AUTO)
    # one element off a 16-byte boundary on both sides
    flat = to_dev(a.reshape(-1))
    buf = torch.empty(a.size + 1, dtype=flat.dtype, device=DEV)
    buf[1:] = flat
    out = torch.empty(a.size + 1, dtype=flat.dtype, device=DEV)
    announce("narrow unaligned", esz, c)
    T.swz_transpose(buf[1:], out[1:], rows, c, esz, "swizzle", kind)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out[1:], a).reshape(c, rows), O.transpose(a))
    # a batch of narrow matrices
    b = GEN[esz](3 * 208, c, seed=c + 1).reshape(3, 208, c)
    for layout in [x for x in LAYOUTS + ["direct"] if x != "pad" or c * esz >= 4]:
        announce("narrow batch", esz, c, layout)
        src = to_dev(b)
        dst = torch.empty((3, c, 208), dtype=src.dtype, device=DEV)
        T.swz_convert_layout(src, dst, 3, 208, c, esz, layout, kind)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst, b), O.convert_layout(b))


@pytest.mark.parametrize("kind,esz,c", NARROW_KINDS)
def test_narrow_any_valid_swizzle(kind, esz, c):
    """Every admissible (B, M, S) of either sign moves data only inside LDS
    (M keeps the 4-byte LDS writes whole: M >= log2(4 / esz))."""
    tr = T.swz_plan(0, 4096, c, esz, "swizzle", kind)["tile"][0]
    a = GEN[esz](2 * tr + 16, c, seed=30 + c)
    rng = np.random.default_rng(c + 100 * esz)
    log_tile = (tr * c).bit_length() - 1
    m_min = {4: 0, 2: 1, 1: 2}[esz]
    triples = [(B, M, S) for B in range(1, 6) for M in range(m_min, 5) for S in range(-9, 10)
               if S != 0 and M + B <= log_tile and (M + B if S > 0 else M - S + B) <= log_tile]
    for idx in rng.choice(len(triples), size=12, replace=False):
        B, M, S = triples[idx]
        for layout in ("swizzle", "direct") if abs(S) >= B else ("swizzle",):
            announce("narrow params", esz, c, layout, (B, M, S))
            check_transpose(a, esz, layout, kind, (B, M, S))


def test_seeded_random_conversions():
    """80 seeded random conversions: element size, batch, rows and columns
    (1-600, so pitches of any alignment, partial tiles and partial stacked
    blocks in both directions), layout and tile order, each through the
    AUTO read kind and compared with the oracle."""
    rng = np.random.default_rng(2026)
    gen = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}
    for case in range(80):
        esz = int(rng.choice([1, 2, 4]))
        b, r, c = int(rng.integers(1, 4)), int(rng.integers(1, 601)), int(rng.integers(1, 601))
        layout = str(rng.choice(["swizzle", "pad", "plain", "direct"]))
        order = int(rng.choice(T.ORDERS))
        a = gen[esz](b * r, c, seed=case).reshape(b, r, c)
        announce("random conversion", case, esz, (b, r, c), layout, order)
        T.swz_set_tile_order(b, r, c, esz, T.READ_AUTO, order)
        try:
            src = to_dev(a)
            dst = torch.empty((b, c, r), dtype=src.dtype, device=DEV)
            try:
                T.swz_convert_layout(src, dst, b, r, c, esz, layout)
            except T.SwzError as e:
                # a direct fill needs 16-byte row pitches; no padded rows narrower than 4 bytes
                assert e.status == T.SWZ_EUNSUPPORTED and layout in ("direct", "pad"), (case, e)
                continue
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(dst, a), O.convert_layout(a)), (case, esz, (b, r, c), layout, order)
        finally:
            T.swz_set_tile_order(b, r, c, esz, T.READ_AUTO, -1)


def test_misaligned_output_rows_through_the_xcd_grouped_grid():
    """Output rows that are not whole 64-byte pieces, from 2,000 rows on,
    run through the XCD-renumbered block grid with cached accesses: every
    element size, batches (the renumbering spans the z dimension), partial
    tiles, padded and plain layouts, pinned orders; plus unaligned pitches
    of every element size (the element path on the same renumbered grid,
    with unaligned vector accesses for 1- and 2-byte elements)."""
    cases = [(1, 2008, 1000, 4), (3, 2056, 136, 4), (2, 2008, 520, 2), (1, 2064, 528, 1), (2, 4104, 264, 4)]
    for b, r, c, esz in cases:
        gen = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}[esz]
        a = gen(b * r, c, seed=r + c).reshape(b, r, c)
        want = O.convert_layout(a)
        for layout in LAYOUTS:
            for order in (None, T.ORDER_DIAGONAL, T.ORDER_SLOPE_32):
                announce("misaligned output rows", (b, r, c, esz), layout, order)
                if order is not None:
                    T.swz_set_tile_order(b, r, c, esz, T.READ_AUTO, order)
                try:
                    src = to_dev(a)
                    dst = torch.empty((b, c, r), dtype=src.dtype, device=DEV)
                    T.swz_convert_layout(src, dst, b, r, c, esz, layout)
                    torch.cuda.synchronize()
                    assert np.array_equal(from_dev(dst, a), want), ((b, r, c, esz), layout, order)
                finally:
                    T.swz_set_tile_order(b, r, c, esz, T.READ_AUTO, -1)
    for r, c, esz in [(2001, 1003, 1), (2002, 1001, 2), (3003, 517, 1), (2001, 333, 4)]:
        gen = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}[esz]
        a = gen(r, c, seed=r)
        announce("unaligned rows", (r, c, esz))
        check_transpose(a, esz, "swizzle", T.READ_AUTO)


def test_rows_kind_every_width():
    """Flat whole-row tiles (SWZ_READ_ROWS, and AUTO for widths that are
    not powers of two): every width up to 128 columns of every element size,
    row counts around the lane-word groups, the 64-byte output line (h
    elements), the tile and its halo, batches, base pointers 0 to h - 1
    elements past a line, both layouts."""
    rng = np.random.default_rng(2028)
    gen = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}
    for esz, cmax in ((4, 128), (2, 128), (1, 128)):
        group, h = 64 * (4 // esz), 64 // esz
        for c in range(1, cmax + 1):
            tr = (16384 if c <= 64 else 32768) // (c * esz) // group * group
            counts = {1, h - 1, h + 1, group - 1, group + 1, tr - 1, tr, tr + 1, tr + h - 1, tr + h + 1,
                      2 * tr + int(rng.integers(1, group))}
            for rows in sorted(counts):
                b = 1 + (c + rows) % 3
                a = gen[esz](b * rows, c, seed=c + rows).reshape(b, rows, c)
                want = O.convert_layout(a)
                for layout, kind, off in (("swizzle", T.READ_ROWS, (7 * c + rows) % h), ("plain", T.READ_AUTO, 1)):
                    if kind == T.READ_AUTO and (c & (c - 1)) == 0:
                        kind = T.READ_ROWS  # AUTO takes the swizzled kinds for powers of two
                    announce("rows kind", esz, (b, rows, c), layout, off)
                    flat = np.concatenate([np.zeros(off, a.dtype), a.reshape(-1)])
                    src = to_dev(flat)
                    dst = torch.zeros(off + a.size, dtype=src.dtype, device=DEV)
                    T.swz_convert_layout(src[off:], dst[off:], b, rows, c, esz, layout, kind)
                    torch.cuda.synchronize()
                    got = from_dev(dst, a)
                    assert np.array_equal(got[off:].reshape(b, c, rows), want), (esz, (b, rows, c), layout, off)
                    assert not got[:off].any()
    # caller-given swizzles of word offsets
    for esz, c in ((4, 12), (2, 6), (2, 24), (1, 48), (1, 10)):
        a = gen[esz](3000, c, seed=c).reshape(1, 3000, c)
        for params in ((1, 0, 5), (3, 0, 6), (5, 0, 11), (0, 0, 0)):
            announce("rows kind params", esz, c, params)
            src = to_dev(a)
            dst = torch.empty((1, c, 3000), dtype=src.dtype, device=DEV)
            T.swz_convert_layout(src, dst, 1, 3000, c, esz, "swizzle", T.READ_ROWS, params)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(dst, a), O.convert_layout(a)), (esz, c, params)


def test_seeded_random_operand_pairs():
    """40 seeded random operand pairs (m, n multiples of 16 up to 592, k a
    multiple of 32 up to 704) staged in one launch in a random layout."""
    rng = np.random.default_rng(2027)
    for case in range(40):
        m, n, k = 16 * int(rng.integers(1, 38)), 16 * int(rng.integers(1, 38)), 32 * int(rng.integers(1, 23))
        layout = str(rng.choice(["swizzle", "pad", "plain", "direct"]))
        announce("random pair", case, (m, n, k), layout)
        a, bt = W.bf16_operands(m, n, k, seed=100 + case)
        fa = torch.empty(a.size, dtype=torch.int16, device=DEV)
        fb = torch.empty(bt.size, dtype=torch.int16, device=DEV)
        T.swz_stage_operands(to_dev(a), fa, m, to_dev(bt), fb, n, k, layout=layout)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(fa, a), O.stage_operand(a).reshape(-1)), (case, m, n, k, layout)
        assert np.array_equal(from_dev(fb, bt), O.stage_operand(bt).reshape(-1)), (case, m, n, k, layout)


# ------------------------------------------------------------ tile orders


@pytest.mark.parametrize("order", T.ORDERS)
def test_every_tile_order_gives_the_transpose(order):
    """Each order visits every tile once: whole and ragged grids, batches,
    and the 1-D launch (a batch beyond the grid's z limit)."""
    cases = [(W.fp32_matrix(3 * 96, 160, seed=40).reshape(3, 96, 160), 4, T.READ_SCALAR_COL),
             (W.fp16_matrix(2 * 130, 200, seed=41).reshape(2, 130, 200), 2, T.READ_B64_TR16),
             (W.u8_matrix(136, 520, seed=42).reshape(1, 136, 520), 1, T.READ_B64_TR8),
             (W.fp32_matrix(70000 * 4, 36, seed=43).reshape(70000, 4, 36), 4, T.READ_SCALAR_COL)]
    for a, esz, kind in cases:
        b, r, c = a.shape
        T.swz_set_tile_order(b, r, c, esz, kind, order)
        try:
            for layout in LAYOUTS:
                announce("tile order", order, a.shape, layout)
                src = to_dev(a)
                dst = torch.empty((b, c, r), dtype=src.dtype, device=DEV)
                T.swz_convert_layout(src, dst, b, r, c, esz, layout, kind)
                torch.cuda.synchronize()
                assert np.array_equal(from_dev(dst, a), O.convert_layout(a)), (order, a.shape, layout)
        finally:
            T.swz_set_tile_order(b, r, c, esz, kind, -1)


def test_tune_tile_order_pins_an_order_and_keeps_the_result():
    a = W.fp32_matrix(2048, 544, seed=44)
    src = to_dev(a)
    dst = torch.empty((544, 2048), dtype=src.dtype, device=DEV)
    announce("tune tile order")
    try:
        chosen = T.swz_tune_tile_order(src, dst, 1, 2048, 544, 4, "swizzle", reps=3)
        assert chosen in T.ORDERS
        assert T.swz_get_tile_order(1, 2048, 544, 4) == chosen
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst, a), O.transpose(a))
        dst.zero_()
        T.swz_transpose(src, dst, 2048, 544, 4, "direct")  # the pinned order serves every layout
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst, a), O.transpose(a))
    finally:
        T.swz_set_tile_order(1, 2048, 544, 4, T.READ_AUTO, -1)


def test_tune_tile_order_batched_16bit_pins_per_shape():
    """The tuner on a batch of ragged fp16 matrices: the pinned order is the
    one for (batch, rows, cols, read kind) only, and the result it leaves,
    and a later call with the pin, are the transposes."""
    a = W.fp16_matrix(3 * 200, 328, seed=45).reshape(3, 200, 328)
    src = to_dev(a)
    dst = torch.empty((3, 328, 200), dtype=src.dtype, device=DEV)
    announce("tune tile order batched fp16")
    defaults = [T.swz_get_tile_order(1, 200, 328, 2, T.READ_B64_TR16),
                T.swz_get_tile_order(3, 200, 328, 2, T.READ_B128_8X8)]
    try:
        chosen = T.swz_tune_tile_order(src, dst, 3, 200, 328, 2, "swizzle", T.READ_B64_TR16, reps=2)
        assert T.swz_get_tile_order(3, 200, 328, 2, T.READ_B64_TR16) == chosen
        assert T.swz_get_tile_order(1, 200, 328, 2, T.READ_B64_TR16) == defaults[0]  # other shapes untouched
        assert T.swz_get_tile_order(3, 200, 328, 2, T.READ_B128_8X8) == defaults[1]
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst, a), O.convert_layout(a))
        dst.zero_()
        T.swz_convert_layout(src, dst, 3, 200, 328, 2, "pad", T.READ_B64_TR16)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst, a), O.convert_layout(a))
    finally:
        T.swz_set_tile_order(3, 200, 328, 2, T.READ_B64_TR16, -1)


def test_tune_tile_order_refusal_pins_nothing():
    """A conversion the library refuses (a direct fill with a 16-bit row
    pitch that is not a multiple of 16 bytes) makes the tuner return that
    error before any launch, and leaves no order pinned for the shape."""
    src = torch.zeros((64, 100), dtype=torch.int16, device=DEV)
    dst = torch.zeros((100, 64), dtype=torch.int16, device=DEV)
    default = T.swz_get_tile_order(1, 64, 100, 2, T.READ_B64_TR16)
    with pytest.raises(T.SwzError) as e:
        T.swz_tune_tile_order(src, dst, 1, 64, 100, 2, "direct", T.READ_B64_TR16, reps=2)
    assert e.value.status == T.SWZ_EUNSUPPORTED
    assert T.swz_get_tile_order(1, 64, 100, 2, T.READ_B64_TR16) == default
    assert not dst.any().item()  # nothing was written


# ------------------------------------------------------- operand staging


@pytest.mark.parametrize("layout", LAYOUTS)
def test_stage_operand_shapes(layout):
    for mn, k in [(16, 32), (256, 64), (272, 96), (512, 4096 // 8), (48, 608)]:
        a, bt = W.bf16_operands(mn, mn, k, seed=mn + k)
        for op in (a, bt):
            announce("stage", layout, mn, k)
            src = to_dev(op)
            frag = torch.empty(op.size, dtype=src.dtype, device=DEV)
            T.swz_stage_operand(src, frag, mn, k, layout=layout)
            torch.cuda.synchronize()
            ref = O.stage_operand(op).reshape(-1)
            assert np.array_equal(from_dev(frag, op), ref), (mn, k, layout)


def test_stage_operand_any_valid_swizzle():
    # k = 320: four whole k tiles in one stacked workgroup, a fifth in a block of its own
    a, _ = W.bf16_operands(272, 16, 320, seed=12)
    src = to_dev(a)
    ref = O.stage_operand(a).reshape(-1)
    for p in [(3, 3, 3), (3, 3, 4), (4, 3, 4), (2, 4, 7), (5, 3, 6), (1, 3, 1)]:
        frag = torch.empty(a.size, dtype=src.dtype, device=DEV)
        T.swz_stage_operand(src, frag, 272, 320, params=p)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(frag, a), ref), p


@pytest.mark.parametrize("layout", LAYOUTS + ["direct"])
def test_stage_operands_pair_in_one_launch(layout):
    """Both operands of a GEMM staged by one call equal each operand's own
    staging: unequal m and n, partial 64 x 64 tiles, a k tail, and one side
    empty (then the call stages the other alone)."""
    for m, n, k in [(272, 48, 96), (256, 512, 64), (48, 272, 608), (16, 16, 32), (0, 272, 96), (272, 0, 96)]:
        announce("stage pair", layout, m, n, k)
        a, bt = W.bf16_operands(max(m, 16), max(n, 16), k, seed=m + 3 * n + k)
        a, bt = a[:m], bt[:n]
        da, db = to_dev(a) if m else None, to_dev(bt) if n else None
        fa = torch.full((max(a.size, 8),), -1, dtype=torch.int16, device=DEV)
        fb = torch.full((max(bt.size, 8),), -1, dtype=torch.int16, device=DEV)
        T.swz_stage_operands(da, fa, m, db, fb, n, k, layout=layout)
        torch.cuda.synchronize()
        if m:
            assert np.array_equal(from_dev(fa, a), O.stage_operand(a).reshape(-1)), (m, n, k, layout)
        else:
            assert (fa == -1).all().item()  # an empty operand is not touched
        if n:
            assert np.array_equal(from_dev(fb, bt), O.stage_operand(bt).reshape(-1)), (m, n, k, layout)
        else:
            assert (fb == -1).all().item()


def test_stage_operands_rejects_overlaps_and_misalignment():
    a, bt = W.bf16_operands(256, 256, 64, seed=3)
    da, db = to_dev(a), to_dev(bt)
    fa = torch.empty(a.size, dtype=torch.int16, device=DEV)
    with pytest.raises(T.SwzError) as e:  # fragments of B written over A's source
        T.swz_stage_operands(da, fa, 256, db, da, 256, 64)
    assert e.value.status == T.SWZ_EINVAL
    with pytest.raises(T.SwzError):  # both fragment buffers the same memory
        T.swz_stage_operands(da, fa, 256, db, fa, 256, 64)
    with pytest.raises(T.SwzError):  # k not a multiple of 32
        T.swz_stage_operands(da, fa, 256, db, torch.empty_like(fa), 256, 48)
    assert T.raw.swz_stage_operands(da.data_ptr() + 2, fa.data_ptr(), 16, db.data_ptr(),
                                    torch.empty_like(fa).data_ptr(), 16, 32, 2, 0, 0, None, None) == T.SWZ_EINVAL
    # the sources may share memory (they are only read)
    fb = torch.empty_like(fa)
    T.swz_stage_operands(da, fa, 256, da, fb, 256, 64)
    torch.cuda.synchronize()
    assert torch.equal(fa, fb)


# --------------------------------------------- full sizes of the workloads


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_fp32_4096(layout):
    announce("full fp32 4096", layout)
    check_transpose(W.fp32_matrix(4096, 4096, seed=0), 4, layout, T.READ_AUTO)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_fp16_8192(layout):
    announce("full fp16 8192", layout)
    check_transpose(W.fp16_matrix(8192, 8192, seed=0), 2, layout, T.READ_B64_4X4)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_fp16_8192_transpose_read(layout):
    announce("full fp16 8192 transpose read", layout)
    check_transpose(W.fp16_matrix(8192, 8192, seed=0), 2, layout, T.READ_B64_TR16)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_u8_8192_transpose_read(layout):
    announce("full u8 8192 transpose read", layout)
    check_transpose(W.u8_matrix(8192, 8192, seed=0), 1, layout, T.READ_B64_TR8)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_bf16_convert(layout):
    announce("full bf16 convert", layout)
    a = W.bf16_tensor((64, 4096, 128), seed=0)
    src = to_dev(a)
    dst = torch.empty((64, 128, 4096), dtype=src.dtype, device=DEV)
    T.swz_convert_layout(src, dst, 64, 4096, 128, 2, layout, T.READ_B128_8X8)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dst, a), O.convert_layout(a))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_full_operand_staging(layout):
    announce("full staging", layout)
    a, bt = W.bf16_operands(8192, 8192, 4096, seed=0)
    for op in (a, bt):
        src = to_dev(op)
        frag = torch.empty(op.size, dtype=src.dtype, device=DEV)
        T.swz_stage_operand(src, frag, op.shape[0], op.shape[1], layout=layout)
        torch.cuda.synchronize()
        got = from_dev(frag, op).reshape(op.shape[0] // 16, op.shape[1] // 32, 64, 8)
        assert np.array_equal(got, O.stage_operand(op))


@pytest.mark.parametrize("layout", LAYOUTS + ["direct"])
def test_full_operand_pair_staging(layout):
    """The staging workload as the benchmark times it: A [8192][4096] and
    B^T [8192][4096] in one launch."""
    announce("full pair staging", layout)
    a, bt = W.bf16_operands(8192, 8192, 4096, seed=0)
    da, db = to_dev(a), to_dev(bt)
    fa, fb = torch.empty_like(da), torch.empty_like(db)
    T.swz_stage_operands(da, fa, 8192, db, fb, 8192, 4096, layout=layout)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(fa, a).reshape(512, 128, 64, 8), O.stage_operand(a))
    assert np.array_equal(from_dev(fb, bt).reshape(512, 128, 64, 8), O.stage_operand(bt))


# ---------------------------------------------------- the reference copy


@pytest.mark.parametrize("layout", LAYOUTS + ["direct"])
def test_full_fp32_narrow8(layout):
    """fp32 [2^21][8] -> [8][2^21] (64 MiB), the narrow-row workload."""
    a = W.fp32_matrix(1 << 21, 8, seed=0)
    announce("full narrow8", layout)
    check_transpose(a, 4, layout, T.READ_AUTO)


@pytest.mark.parametrize("esz,c", [(2, 8), (1, 16)])
@pytest.mark.parametrize("layout", ["swizzle", "direct"])
def test_full_small_narrow(esz, c, layout):
    """fp16 [2^22][8] and u8 [2^22][16] (64 MiB each), whole-row tiles of
    2- and 1-byte elements."""
    a = GEN[esz](1 << 22, c, seed=1)
    announce("full small narrow", esz, c, layout)
    check_transpose(a, esz, layout, T.READ_AUTO)


def test_reference_copy():
    """swz_copy (the bandwidth ceiling the kernels are compared with, and the
    byte-counter scale) moves every byte, for sizes with and without a
    partial workgroup."""
    for nbytes in (16, 4096 + 48, 64 * 2**20, 64 * 2**20 + 16 * 37):
        announce("copy", nbytes)
        src = torch.randint(-128, 128, (nbytes,), dtype=torch.int8, device=DEV)
        dst = torch.zeros_like(src)
        T.swz_copy(src, dst, nbytes)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), nbytes


@pytest.mark.parametrize("esz", [4, 2, 1])
def test_offset_pointers_through_the_xcd_grouped_grid(esz):
    """Both pointers 1 to 32 bytes past a 64-byte line (element multiples),
    from 2,000 rows: every output row then starts off the 64-byte pieces, so
    the launches take the XCD-grouped grid (aligned block grid for 16 and 32
    bytes, the element path's for the others; bytes 1 and 2 bytes off keep
    the plain grid), on matrices with edge tiles and of whole tiles only;
    every layout of the register fill."""
    kind = {4: T.READ_SCALAR_COL, 2: T.READ_B64_TR16, 1: T.READ_B64_TR8}[esz]
    shapes = ((2048, 2048), (2051, 1000)) if esz == 4 else ((2048, 2048), (2083, 700))
    for rows, cols in shapes:
        a = GEN[esz](rows, cols, seed=rows + cols + esz)
        want = O.transpose(a)
        flat = a.reshape(-1)
        for off in sorted({1, 2, 4, 16, 32} - {1, 2} if esz == 4 else {1, 2, 4, 16, 32} - ({1} if esz == 2 else set())):
            n = off // esz  # elements before the matrix in both buffers
            for layout in LAYOUTS:
                announce("offset pointers", esz, (rows, cols), off, layout)
                src = to_dev(np.concatenate([np.zeros(n + 64 // esz, a.dtype), flat]))
                dst = torch.zeros_like(src)
                s0 = 64 // esz + n  # 64 bytes in, then the offset
                T.swz_transpose(src[s0:], dst[s0:], rows, cols, esz, layout, kind)
                torch.cuda.synchronize()
                got = from_dev(dst, a)
                assert np.array_equal(got[s0:].reshape(cols, rows), want), (esz, (rows, cols), off, layout)
                assert not got[:s0].any()
