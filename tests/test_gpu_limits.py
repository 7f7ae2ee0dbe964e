"""Launch-shape limits (needs a GPU): grids beyond the hardware's 3-D limits
take the 1-D chunked launch path, and jobs above 2^22 tiles are split over
several launches.  Outputs are compared with the oracle on whole batch
entries or row blocks sampled at the start, at the chunk boundary and at
the end.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W

import torch  # noqa: E402  (hard imports: a GPU run without them fails, never skips)

import tiled_movement_amd as T  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(*what):
    print("case:", *what, flush=True)


def test_transpose_with_more_tile_columns_than_a_grid_dimension():
    rows, cols = 40, 32 * 65537 + 8  # 65,538 tile columns > 65,535
    a = W.fp32_matrix(rows, cols, seed=40)
    for layout in ("swizzle", "direct"):
        announce("wide transpose", layout, rows, cols)
        src = torch.from_numpy(a.view(np.int32)).to(DEV)
        dst = torch.empty((cols, rows), dtype=torch.int32, device=DEV)
        T.swz_transpose(src, dst, rows, cols, 4, layout)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy().view(np.uint32), O.transpose(a))


def test_transpose_whose_tile_blocks_overflow_a_grid_dimension():
    """16-bit rows of 65,536 tiles of 64 (the last one partial): the blocks
    of the one-launch grid would need 65,536 workgroups along y, so the
    whole tiles go through the interior launch and the partial column
    through the 1-D edge launch."""
    rows, cols = 128, 64 * 65535 + 8
    a = W.fp16_matrix(rows, cols, seed=41)
    want = O.transpose(a)
    for layout in ("swizzle", "direct"):
        announce("wide 16-bit transpose", layout, rows, cols)
        src = torch.from_numpy(a.view(np.int16)).to(DEV)
        dst = torch.empty((cols, rows), dtype=torch.int16, device=DEV)
        T.swz_transpose(src, dst, rows, cols, 2, layout)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy().view(np.uint16), want.view(np.uint16))
    del src, dst
    torch.cuda.empty_cache()


def test_batch_beyond_grid_limit_and_more_than_2_22_tiles():
    """65,537 batch entries of 256 x 256 fp32 = 4,194,368 tiles of 32 x 32:
    a batch beyond the 65,535 grid limit and one tile chunk past 2^22."""
    batch, rows, cols = 65537, 256, 256  # 2 x 34 GB: fits in one MI355X's 288 GB
    announce("huge batch", batch, rows, cols)
    src = W.index_pattern_device((batch, rows, cols), DEV, 4)
    dst = torch.empty((batch, cols, rows), dtype=torch.int32, device=DEV)
    T.swz_convert_layout(src, dst, batch, rows, cols, 4, "swizzle")
    torch.cuda.synchronize()
    tiles_per_entry = (rows // 32) * (cols // 32)
    boundary = (1 << 22) // tiles_per_entry  # first entry of the second launch chunk
    for b in sorted({0, 1, 12345, boundary - 1, boundary, batch - 1}):
        a = W.index_pattern_host((batch, rows, cols), b, 4)
        got = dst[b].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, O.transpose(a)), b
    del src, dst
    torch.cuda.empty_cache()


def test_stage_with_more_row_tiles_than_a_grid_dimension():
    mn, k = 64 * 65537, 64  # 65,537 row tiles of 64 > 65,535
    announce("tall staging", mn, k)
    src = W.index_pattern_device((mn // 16, 16 * k), DEV, 2)  # rows of 16 x k, same bytes as [mn][k]
    frag = torch.empty(mn * k, dtype=torch.int16, device=DEV)
    for layout in ("swizzle", "direct"):
        frag.zero_()
        T.swz_stage_operand(src, frag, mn, k, layout=layout)
        torch.cuda.synchronize()
        f = frag.view(mn // 16, k // 32, 64, 8)
        tile0 = [W.index_pattern_host((mn // 16, 16 * k), b, 2) for b in range(4)]  # row blocks of tile 0
        for blk in sorted({0, 3, 4 * 65535, 4 * 65536 + 3, mn // 16 - 1}):
            x = W.index_pattern_host((mn // 16, 16 * k), blk, 2).reshape(16, k)
            if blk >= 4:  # a read of tile 0's rows for this block would show
                assert not any(np.array_equal(x.reshape(-1), t) for t in tile0), blk
            got = f[blk].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, O.stage_operand(x)[0]), (layout, blk)


@pytest.mark.parametrize("esz,c", [(4, 8), (2, 1), (2, 32), (1, 4), (1, 64)])
def test_narrow_rows_batch_beyond_grid_limit(esz, c):
    """70,000 small narrow-row matrices: a batch beyond the 65,535 grid limit
    takes the 1-D launch, with whole-row tiles of every element size."""
    batch, rows = 70000, 24
    gen = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}[esz]
    a = gen(batch * rows, c, seed=50 + c).reshape(batch, rows, c)
    for layout in ("swizzle", "plain"):
        announce("narrow huge batch", esz, c, layout)
        src = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        dst = torch.empty((batch, c, rows), dtype=src.dtype, device=DEV)
        T.swz_convert_layout(src, dst, batch, rows, c, esz, layout)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy(), O.convert_layout(a)), (esz, c, layout)


@pytest.mark.parametrize("esz,c", [(4, 3), (1, 48), (2, 66)])
def test_rows_kind_more_than_2_22_tiles(esz, c):
    """2^22 + 3 entries of 2 rows, one flat-row tile each: more tiles than one
    launch takes, so the tile numbering carries across launch chunks (bytes
    x 48 and 2-byte x 66 with runs shifted onto the output lines, the latter
    in 512-thread tiles)."""
    batch, rows = (1 << 22) + 3, 2
    gen = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}[esz]
    a = gen(batch * rows, c, seed=60 + c).reshape(batch, rows, c)
    announce("rows kind past 2^22 tiles", esz, c)
    src = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    dst = torch.empty((batch, c, rows), dtype=src.dtype, device=DEV)
    T.swz_convert_layout(src, dst, batch, rows, c, esz, "swizzle", T.READ_ROWS)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), O.convert_layout(a)), (esz, c)
    del src, dst
    torch.cuda.empty_cache()


def test_rows_kind_at_the_timed_sizes():
    """The flat-row transposes the benchmark times, whole: fp32 [5592405][3]
    (unshifted runs) and bytes [1398101][48] (runs shifted onto the output
    lines), both layouts, compared element by element with the oracle."""
    for esz, c, gen in ((4, 3, W.fp32_matrix), (1, 48, W.u8_matrix)):
        r = (64 << 20) // (c * esz)
        a = gen(r, c, seed=0)
        want = O.transpose(a)
        for layout in ("swizzle", "plain"):
            announce("rows kind, timed size", esz, (r, c), layout)
            src = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
            dst = torch.empty((c, r), dtype=src.dtype, device=DEV)
            T.swz_convert_layout(src, dst, 1, r, c, esz, layout, T.READ_ROWS)
            torch.cuda.synchronize()
            assert np.array_equal(dst.cpu().numpy(), want), (esz, c, layout)
