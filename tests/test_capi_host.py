"""Host-side checks of libswz.so (no GPU needed).

* the library loads and exports every function include/swz.h declares;
* argument validation returns the documented codes before any launch;
* the kernels' LDS access patterns equal an independent restatement of the
  lane maps, with addresses computed by the oracle's swizzle;
* the library's conflict predictor agrees with the oracle's brute-force
  counter under the same bank model, and its chooser with the oracle's.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

import tiled_movement_amd as T  # noqa: E402  (the library must be built: no skip)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swz.h")
lib = T.lib
P = T.Params
EINVAL, EUNSUP = T.SWZ_EINVAL, T.SWZ_EUNSUPPORTED


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(swz_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(T.EXPORTS)


def test_strerror():
    assert T.strerror(0) == "ok"
    assert "invalid" in T.strerror(EINVAL)
    assert T.strerror(12345) == "unknown status"


# ------------------------------------------------------ argument checking
# Fake, never-dereferenced device addresses: every call below must be
# rejected (or be a no-op) before anything reaches the HIP runtime.
A, B, C = 0x7F0000000000, 0x7F0100000000, 0x7F0200000000


def test_map_validation():
    assert lib.swz_map(A, B, -1, P(1, 0, 1), None) == EINVAL
    assert lib.swz_map(A, B, 16, P(-1, 0, 1), None) == EINVAL
    assert lib.swz_map(A, B, 16, P(5, 20, 8), None) == EINVAL  # fields leave 32 bits
    assert lib.swz_map(None, B, 16, P(1, 0, 1), None) == EINVAL
    assert lib.swz_map(A + 2, B, 16, P(1, 0, 1), None) == EINVAL  # not 4-byte aligned
    assert lib.swz_map(A, A + 8, 16, P(1, 0, 1), None) == EINVAL  # partial overlap
    assert lib.swz_map(A, B, 0, P(1, 0, 1), None) == T.SWZ_OK  # nothing to do


def test_map_batch_validation():
    f = lib.swz_map_batch
    good = (P * 3)(P(1, 0, 1), P(3, 1, -4), P(0, 0, 0))
    bad = (P * 3)(P(1, 0, 1), P(5, 20, 8), P(0, 0, 0))  # the second triple leaves 32 bits
    assert f(A, B, -1, good, 3, None) == EINVAL
    assert f(A, B, 16, good, -1, None) == EINVAL
    assert f(A, B, 16, None, 3, None) == EINVAL
    assert f(A, B, 16, bad, 3, None) == EINVAL  # refused before any launch
    assert f(None, B, 16, good, 3, None) == EINVAL
    assert f(A + 2, B, 16, good, 3, None) == EINVAL  # not 4-byte aligned
    assert f(A, A + 32, 16, good, 3, None) == EINVAL  # output rows overlap the input
    assert f(A + 128, A, 16, good, 3, None) == EINVAL  # input inside the second output row
    assert f(A, B, 0, good, 3, None) == T.SWZ_OK  # nothing to do
    assert f(A, B, 16, None, 0, None) == T.SWZ_OK
    assert f(A, B, 1 << 62, good, 3, None) == EINVAL  # size overflow


def test_tile_order_validation():
    f = lib.swz_set_tile_order
    assert f(-1, 64, 64, 4, -1, 0) == EINVAL
    assert f(1, 64, 64, 4, -1, 7) == EINVAL  # no such order
    assert f(1, 64, 64, 4, -1, -2) == EINVAL
    assert f(1, 64, 64, 3, -1, 0) == EINVAL  # element size
    assert f(1, 64, 64, 2, T.READ_SCALAR_COL, 0) == EINVAL  # kind for another element size
    assert f(1, 64, 1024, 4, -1, T.ORDER_COLUMNS) == T.SWZ_OK
    assert T.swz_get_tile_order(1, 64, 1024, 4) == T.ORDER_COLUMNS
    assert T.swz_get_tile_order(1, 64, 1024, 4, T.READ_SCALAR_COL) == T.ORDER_COLUMNS  # AUTO resolves to this kind
    assert T.swz_get_tile_order(2, 64, 1024, 4) == T.ORDER_DIAGONAL  # another shape
    assert lib.swz_get_tile_order(1, 64, 1024, 4, -1, None) == EINVAL
    assert f(1, 64, 1024, 4, -1, -1) == T.SWZ_OK  # removed
    assert T.swz_get_tile_order(1, 64, 1024, 4) == T.ORDER_DIAGONAL
    assert f(1, 64, 1024, 4, -1, -1) == T.SWZ_OK  # removing twice is fine
    g = lib.swz_tune_tile_order
    c = ctypes.c_int32(-7)
    assert g(A, B, 1, 64, 64, 4, 0, -1, None, 10, None, None) == EINVAL  # no output for the choice
    assert g(A, B, 1, 64, 64, 4, 0, -1, None, 0, ctypes.byref(c), None) == EINVAL  # reps
    assert g(A, B, 1, 64, 64, 4, 0, -1, None, 1001, ctypes.byref(c), None) == EINVAL
    assert g(A, B, 1, 64, 64, 3, 0, -1, None, 10, ctypes.byref(c), None) == EINVAL  # element size
    assert g(A, B, 0, 64, 1024, 4, 0, -1, None, 10, ctypes.byref(c), None) == T.SWZ_OK  # nothing to time
    assert c.value == T.ORDER_DIAGONAL
    assert g(A, B, 0, 64, 64, 4, 0, -1, None, 10, ctypes.byref(c), None) == T.SWZ_OK
    assert c.value == T.ORDER_SLOPE_32  # the shape's default
    for order in T.ORDERS:
        assert f(1, 96, 64, 4, -1, order) == T.SWZ_OK
        assert T.swz_get_tile_order(1, 96, 64, 4) == order
    assert f(1, 96, 64, 4, -1, -1) == T.SWZ_OK


def test_default_tile_order_by_shape():
    """Unpinned shapes: whole tile columns when the output rows (rows x
    element bytes) are not whole 64-byte pieces, there are at least 2,000
    rows and the matrix is at least 16 tiles wide (slope 1/32 when it is
    narrower); else slope 1/32 when the source row pitch (cols x element bytes) is
    not within 1% of a multiple of 4 KiB; otherwise the diagonal, or slope
    1/8 for fp32 matrices with at most 10,240 rows and a side that is not a
    power of two.  Whole-row kinds: the diagonal."""
    get = T.swz_get_tile_order
    # pitch a multiple of 4 KiB
    assert get(1, 4096, 4096, 4) == T.ORDER_DIAGONAL
    assert get(1, 8192, 2048, 4) == T.ORDER_DIAGONAL
    assert get(7, 3072, 4096, 4) == T.ORDER_SLOPE_8  # per batch entry
    assert get(1, 10240, 3072, 4) == T.ORDER_SLOPE_8
    assert get(1, 10256, 3072, 4) == T.ORDER_DIAGONAL  # over 10,240 rows (output rows whole 64-byte pieces)
    assert get(1, 12288, 4096, 4) == T.ORDER_DIAGONAL
    assert get(1, 8192, 8192, 2) == T.ORDER_DIAGONAL
    assert get(1, 5760, 6144, 2) == T.ORDER_DIAGONAL
    # within 1% of a multiple: fp32 8128 columns (32,512 bytes, 256 below 32 KiB), 16-bit 8128 (128 below)
    assert get(1, 5760, 8128, 4) == T.ORDER_SLOPE_8
    assert get(1, 16384, 8128, 4) == T.ORDER_DIAGONAL
    assert get(1, 5760, 8128, 2) == T.ORDER_DIAGONAL
    # further off: 16-bit 4160 columns (8,320 bytes: 128 over 8 KiB is 1.5%), fp32 5760, 3000
    assert get(1, 5760, 4160, 2) == T.ORDER_SLOPE_32
    assert get(1, 5760, 5760, 4) == T.ORDER_SLOPE_32
    assert get(1, 4096, 5760, 4, T.READ_SCALAR_COL) == T.ORDER_SLOPE_32
    assert get(1, 16384, 3000, 4) == T.ORDER_SLOPE_32  # whatever the rows
    assert get(1, 5760, 5760, 2) == T.ORDER_SLOPE_32
    assert get(1, 8192, 512, 2) == T.ORDER_SLOPE_32  # rows of 1 KiB
    # bytes: the same rule on the 8-bit transpose-read kind; whole-row kinds keep the diagonal
    assert get(1, 5760, 5760, 1) == T.ORDER_SLOPE_32
    # output rows (rows x element bytes) off the 64-byte pieces, from 2,000 rows: whole tile columns
    assert get(1, 5800, 5800, 4) == T.ORDER_COLUMNS
    assert get(3, 3000, 4096, 4) == T.ORDER_COLUMNS
    assert get(1, 2008, 8192, 4) == T.ORDER_COLUMNS
    assert get(1, 1000, 8192, 4) == T.ORDER_SLOPE_8  # fewer rows: the pitch rules
    assert get(1, 5760, 5800, 4) == T.ORDER_SLOPE_32  # only the source pitch is off
    assert get(1, 4112, 4112, 2) == T.ORDER_COLUMNS
    assert get(1, 8208, 8208, 1) == T.ORDER_COLUMNS
    assert get(1, 8208, 16, 1) == T.ORDER_DIAGONAL  # whole-row kind
    # ... unless the matrix is under 16 tiles wide (32-, 64- and 128-column tiles): slope 1/32
    assert get(1, 223696, 300, 1) == T.ORDER_SLOPE_32  # 3 tiles of 128 columns
    assert get(1, 67108, 500, 2) == T.ORDER_SLOPE_32  # 8 of 64
    assert get(1, 55924, 300, 4) == T.ORDER_SLOPE_32  # 10 of 32
    assert get(1, 33554, 500, 4) == T.ORDER_COLUMNS  # 16 of 32
    assert get(1, 33554, 1000, 2) == T.ORDER_COLUMNS  # 16 of 64
    assert get(1, 33554, 2048, 1) == T.ORDER_COLUMNS  # 16 of 128
    assert get(1, 8192, 8192, 1) == T.ORDER_DIAGONAL
    assert get(1, 5760, 8128, 1) == T.ORDER_DIAGONAL  # 64 bytes short of 8 KiB
    assert get(1, 5760, 4160, 1) == T.ORDER_SLOPE_32  # 64 over 4 KiB: 1.5%
    assert get(1, 1 << 20, 16, 1) == T.ORDER_DIAGONAL  # one tile column
    assert get(1, 1 << 20, 8, 4) == T.ORDER_DIAGONAL


def test_convert_validation():
    f = lib.swz_convert_layout
    assert f(A, B, 1, 64, 64, 3, 0, -1, None, None) == EINVAL  # element size
    assert f(A, B, -1, 64, 64, 4, 0, -1, None, None) == EINVAL
    assert f(A, B, 1, -64, 64, 4, 0, -1, None, None) == EINVAL
    assert f(A, B, 1, 64, 64, 4, 7, -1, None, None) == EINVAL  # layout
    assert f(A, B, 1, 64, 64, 2, 0, T.READ_SCALAR_COL, None, None) == EINVAL  # kind vs size
    assert f(A, B, 1, 64, 64, 4, 0, T.READ_B64_4X4, None, None) == EINVAL
    assert f(A, B, 1, 64, 64, 2, 0, T.READ_MFMA_16X16X32, None, None) == EINVAL
    assert f(A, B, 1, 64, 64, 2, 0, 9, None, None) == EINVAL
    bad = [P(3, 2, 3), P(5, 3, 0), P(5, 9, 3), P(-1, 3, 3), P(20, 3, 20)]
    for p in bad:  # splits a 16-byte vector / S = 0 / leaves the tile / negative / too wide
        assert f(A, B, 1, 64, 64, 2, 0, T.READ_B64_4X4, ctypes.byref(p), None) == EINVAL, p.tuple()
    assert f(A, A + 64, 1, 64, 64, 4, 0, -1, None, None) == EINVAL  # overlap
    assert f(A + 2, B, 1, 64, 64, 4, 0, -1, None, None) == EINVAL  # not element aligned
    assert f(None, B, 1, 64, 64, 4, 0, -1, None, None) == EINVAL
    assert f(A, B, 1 << 40, 1 << 20, 1 << 20, 4, 0, -1, None, None) == EINVAL  # size overflow
    for shape in [(0, 64, 64), (3, 0, 64), (3, 64, 0)]:
        assert f(A, B, *shape, 4, 0, -1, None, None) == T.SWZ_OK  # empty: no launch
    # an empty batch with rows whose byte pitch exceeds int64: checked without overflow
    assert f(A, B, 0, (1 << 63) - 1, 8, 4, 0, -1, None, None) == T.SWZ_OK
    assert f(A, B, 0, 8, (1 << 63) - 1, 4, 0, T.READ_SCALAR_COL, None, None) == T.SWZ_OK
    assert lib.swz_transpose(A, B, 64, 64, 8, 0, -1, None, None) == EINVAL


def test_stage_validation():
    f = lib.swz_stage_operand
    assert f(A, B, 17, 64, 2, 0, 0, None, None) == EINVAL  # partial fragment rows
    assert f(A, B, 16, 48, 2, 0, 0, None, None) == EINVAL  # partial fragment k
    assert f(A, B, 16, 32, 4, 0, 0, None, None) == EINVAL  # element size
    assert f(A, B, 16, 32, 2, 1, 0, None, None) == EINVAL  # fragment kind
    assert f(A + 8, B, 16, 32, 2, 0, 0, None, None) == EINVAL  # 16-byte alignment
    assert f(A, A + 16, 16, 32, 2, 0, 0, None, None) == EINVAL  # overlap
    assert f(A, B, 16, 32, 2, 0, 0, ctypes.byref(P(3, 2, 3)), None) == EINVAL
    assert f(A, B, 0, 32, 2, 0, 0, None, None) == T.SWZ_OK


def test_probe_and_query_validation():
    c = ctypes.c_int64()
    assert lib.swz_lds_probe(A, B, 4, 3, 0, 8, 4, A + 4096, None) == EINVAL
    assert lib.swz_lds_probe(A, B, 4, 4, 0, 8, 17, A + 4096, None) == EINVAL
    assert lib.swz_lds_probe(A, B, 4, 4, 2, 8, 4, A + 4096, None) == EINVAL
    assert lib.swz_lds_probe(A, B, 4, 4, 0, 0, 4, A + 4096, None) == EINVAL
    assert lib.swz_lds_probe(A, B, 0, 4, 0, 8, 4, A + 4096, None) == T.SWZ_OK
    assert lib.swz_predict_conflicts(24, 0, None, ctypes.byref(c), ctypes.byref(c)) == EINVAL  # no such kind
    assert lib.swz_choose(2, 16, 64, 64, 24, ctypes.byref(P())) == EINVAL  # no such kind
    assert lib.swz_choose(2, 16, 64, 32, T.READ_B64_4X4, ctypes.byref(P())) == EUNSUP
    assert lib.swz_bank_model_get(None) == EINVAL
    with pytest.raises(T.SwzError):
        T.swz_plan(1, 17, 64, 2)


def test_plans():
    p = T.swz_plan(0, 4096, 4096, 4, "swizzle")
    assert p["read_kind"] == T.READ_SCALAR_COL and p["tile"] == (32, 32) and p["lds_bytes"] == 4096
    assert T.swz_plan(0, 4096, 4096, 4, "pad")["lds_bytes"] == 32 * 33 * 4
    assert T.swz_plan(0, 8192, 8192, 2)["read_kind"] == T.READ_B64_4X4
    assert T.swz_plan(0, 4096, 128, 2)["read_kind"] == T.READ_B128_8X8
    assert T.swz_plan(0, 64, 64, 2, "pad", T.READ_B64_4X4)["lds_bytes"] == 64 * 72 * 2
    assert T.swz_plan(0, 64, 64, 2, "plain", T.READ_B64_4X4)["params"] == (0, 0, 0)
    s = T.swz_plan(1, 8192, 4096, 2)
    assert s["read_kind"] == T.READ_MFMA_16X16X32 and s["tile"] == (64, 64) and s["threads"] == 256
    # tiles per workgroup of the whole-tile launch
    assert s["interior_tiles"] == 4 and p["interior_tiles"] == 4  # staging: 4 along k; fp32: 2 x 2
    assert T.swz_plan(0, 8192, 8192, 2)["interior_tiles"] == 2
    assert T.swz_plan(0, 4096, 128, 2)["interior_tiles"] == 1
    assert T.swz_plan(0, 64, 64, 2, "swizzle", T.READ_B64_4X4, (3, 3, 6))["params"] == (3, 3, 6)


# ---------------------------------------- lane maps, restated independently
# Which tile element (row, col) lane l of wave w touches at step i, as the
# design describes each kernel; coordinates are of the first element.


NARROW4 = (T.READ_NARROW1, T.READ_NARROW2, T.READ_NARROW4, T.READ_NARROW8, T.READ_NARROW16)
NARROW2 = (T.READ_HNARROW1, T.READ_HNARROW2, T.READ_HNARROW4, T.READ_HNARROW8, T.READ_HNARROW16, T.READ_HNARROW32)
NARROW1 = (T.READ_BNARROW1, T.READ_BNARROW2, T.READ_BNARROW4, T.READ_BNARROW8, T.READ_BNARROW16, T.READ_BNARROW32,
           T.READ_BNARROW64)
NARROW = NARROW4 + NARROW2 + NARROW1
NO_PAD = (T.READ_HNARROW1, T.READ_BNARROW1, T.READ_BNARROW2)  # rows under one 4-byte LDS store


def plan_cols(kind):
    """A width the kind accepts: narrow kinds take exactly their row width."""
    return KIND_GEOM[kind][2] if kind in NARROW else 4096


def threads_of(kind):
    op = 1 if kind == T.READ_MFMA_16X16X32 else 0
    esz = KIND_GEOM[kind][0]
    return T.swz_plan(op, 4096, plan_cols(kind), esz, "swizzle", kind)["threads"]


def restated_accesses(kind, write):
    """The kernels' lane maps as the design states them: thread t of NT
    handles 16-byte global vector v = t + NT*j and output piece u = t + NT*j."""
    nt = threads_of(kind)
    out = []
    for w in range(nt // 64):
        ts = [64 * w + l for l in range(64)]
        if kind in NARROW:  # tile of whole rows of C elements of esz bytes
            esz_, tr_, c_, _ = KIND_GEOM[kind]
            per, epw = 16 // esz_, 4 // esz_  # elements per 16 bytes / per 4-byte word
            words = esz_ != 2 or c_ == 1 or c_ >= 32  # read back as words, else element by element
            cb = min(c_, epw) if words else 1  # columns per lane block
            rpw = max(1, epw // c_) if words else 1  # whole rows per load
            if write:  # vector v = t + nt*j: flat elements per*v .., one 4-byte word per store:
                # word e, or e ^ (bits 3-4 of the lane) for elements under 4 bytes in rows of 16 or more
                swap = words and esz_ < 4 and c_ >= 16
                for j in range(cb):
                    for e in range(4):
                        coords = [divmod(per * (t + nt * j) + (e ^ ((t >> 3) & 3 if swap else 0)) * epw, c_)
                                  for t in ts]
                        out.append((coords, 4))
            else:  # lane t: rows per*(t % (TR/per)) .., columns cb*(t // (TR/per)) .., one word (element) per load
                blocks = tr_ // per
                for i in range(per // rpw):
                    coords = [(per * (t % blocks) + rpw * i, cb * (t // blocks)) for t in ts]
                    out.append((coords, 4 if words else esz_))
        elif kind == T.READ_SCALAR_COL:  # 32x32 4-byte tile
            for j in range(256 // nt):
                for e in range(4):
                    if write:  # vector v: row v/8, columns 4(v%8)..+3, one element per store
                        coords = [((t + nt * j) // 8, 4 * ((t + nt * j) % 8) + e) for t in ts]
                    else:  # piece u: column u/8, rows 4(u%8)..+3, one row per load
                        coords = [(4 * ((t + nt * j) % 8) + e, (t + nt * j) // 8) for t in ts]
                    out.append((coords, 4))
        elif kind in (T.READ_B64_4X4, T.READ_B128_8X8):
            chunks = 8 if kind == T.READ_B64_4X4 else 16  # 16-byte chunks per row
            tile_rows = 64
            if write:
                for j in range(tile_rows * chunks // nt):
                    coords = [((t + nt * j) // chunks, 8 * ((t + nt * j) % chunks)) for t in ts]
                    out.append((coords, 16))
            else:
                width = 8 if kind == T.READ_B64_4X4 else 16
                for j in range(128 // nt):
                    for s_ in range(8):
                        coords = [(8 * ((t + nt * j) % 8) + s_, (width // 2) * ((t + nt * j) // 8)) for t in ts]
                        out.append((coords, width))
        elif kind == T.READ_B64_TR8:  # 128x128 1-byte tile, 8-bit transpose reads
            if write:  # vector v: row v/8, bytes 16(v%8)..; step h writes half h ^ (row odd)
                for j in range(128 * 128 // 16 // nt):
                    for h in range(2):
                        coords = []
                        for t in ts:
                            v = t + nt * j
                            coords.append((v // 8, 16 * (v % 8) + 8 * (h ^ ((v // 8) % 2))))
                        out.append((coords, 8))
            else:
                # group g (16 lanes) of the wave: loader q addresses row
                # 64h + 16g + 8(q%2) + q//2 of the 8-byte column block
                for k in range(16 // (nt // 64)):
                    ch = w + (nt // 64) * k
                    for h in range(2):
                        coords = []
                        for l in range(64):
                            g, q = divmod(l, 16)
                            coords.append((64 * h + 16 * g + 8 * (q % 2) + q // 2, 8 * ch))
                        out.append((coords, 8))
        elif kind == T.READ_B64_TR16:  # 64x64 2-byte tile, transpose reads
            if write:
                for j in range(4096 * 2 // 16 // nt):
                    coords = [((t + nt * j) // 8, 8 * ((t + nt * j) % 8)) for t in ts]
                    out.append((coords, 16))
            else:
                # group g = lanes 16g..16g+15 covers rows 16g..16g+15 of one
                # 8-column chunk; loader q addresses row 16g + 8*((q%4)//2) +
                # 4*h + q//4 at column 8*chunk + 4*(q%2), h = step ^ (g odd)
                for k in range(8 // (nt // 64)):
                    ch = w + (nt // 64) * k
                    for step in range(2):
                        coords = []
                        for l in range(64):
                            g, q = divmod(l, 16)
                            h = step ^ (g % 2)
                            coords.append((16 * g + 8 * ((q % 4) // 2) + 4 * h + q // 4, 8 * ch + 4 * (q % 2)))
                        out.append((coords, 8))
        else:  # operand staging, 64x64 tile: 4 row blocks x 2 k steps of fragments
            if write:
                for j in range(64 * 8 // nt):
                    coords = [((t + nt * j) // 8, 8 * ((t + nt * j) % 8)) for t in ts]
                    out.append((coords, 16))
            else:
                for i in range(8 // (nt // 64)):
                    f = w + (nt // 64) * i
                    coords = [(16 * (f % 4) + l % 16, 32 * (f // 4) + 8 * (l // 16)) for l in range(64)]
                    out.append((coords, 16))
    return out


KIND_GEOM = {
    T.READ_SCALAR_COL: (4, 32, 32, 1),
    T.READ_B64_4X4: (2, 64, 64, 8),
    T.READ_B128_8X8: (2, 64, 128, 8),
    T.READ_MFMA_16X16X32: (2, 64, 64, 8),
    T.READ_B64_TR16: (2, 64, 64, 8),
    T.READ_B64_TR8: (1, 128, 128, 8),
    T.READ_NARROW1: (4, 1024, 1, 1),
    T.READ_NARROW2: (4, 512, 2, 1),
    T.READ_NARROW4: (4, 256, 4, 1),
    T.READ_NARROW8: (4, 128, 8, 1),
    T.READ_NARROW16: (4, 64, 16, 1),
    # tile rows from the plan: NT lanes, each a block of 16 bytes of rows x min(C, elements per word) columns
    **{k: (2, T.swz_plan(0, 4096, c, 2, "swizzle", k)["tile"][0], c, 2) for k, c in zip(NARROW2, (1, 2, 4, 8, 16, 32))},
    **{k: (1, T.swz_plan(0, 4096, c, 1, "swizzle", k)["tile"][0], c, 4) for k, c in zip(NARROW1, (1, 2, 4, 8, 16, 32, 64))},
}


def oracle_model():
    """The library's built-in bank model rebuilt as an oracle LdsModel."""
    m = T.swz_bank_model_get()
    read, write = {}, {}
    for (dname, width), g in m.items():
        groups = {}
        for lane, ph in enumerate(g["phase"]):
            groups.setdefault(ph, []).append(lane)
        bm = O.BankModel(g["n_banks"], g["bank_bytes"], 64, {width: [groups[k] for k in sorted(groups)]})
        (read if dname == "read" else write)[width] = bm
    # Reading: 1- and 2-byte loads are served like 4-byte ones, lanes that
    # touch the same 4-byte word sharing it (the library's model does this).
    for w in (1, 2):
        read[w] = O.BankModel(read[4].n_banks, read[4].bank_bytes, 64, {w: read[4].phase_groups(4)})
    return O.LdsModel(read, write)


LAYOUT_CASES = [("swizzle", None), ("pad", None), ("plain", None), ("swizzle", "alt")]


@pytest.mark.parametrize("kind", list(KIND_GEOM))
@pytest.mark.parametrize("layout,params", LAYOUT_CASES)
def test_kernel_accesses_match_restated_lane_maps(kind, layout, params):
    esz, tr, tc, pad = KIND_GEOM[kind]
    if layout == "pad" and kind in NO_PAD:
        with pytest.raises(T.SwzError):
            T.swz_kernel_accesses(kind, layout, None, 1)
        return
    if params == "alt":
        params = (3, 0, 6) if esz == 4 else (3, 3, 6)
    chosen = T.swz_plan(1 if kind == T.READ_MFMA_16X16X32 else 0, 4096, plan_cols(kind), esz, layout, kind,
                        params)["params"]
    for write in (1, 0):
        lib_acc = T.swz_kernel_accesses(kind, layout, params, write)
        mine = restated_accesses(kind, write)
        assert len(lib_acc) == len(mine)
        for (addrs, width), (coords, w2) in zip(lib_acc, mine):
            assert width == w2
            expect = O.access_addresses(coords, width // esz, tc, esz, layout, chosen, pad)
            assert addrs == expect


@pytest.mark.parametrize("kind", list(KIND_GEOM))
@pytest.mark.parametrize("layout", ["swizzle", "pad", "plain"])
def test_predictor_matches_oracle_counter(kind, layout):
    if layout == "pad" and kind in NO_PAD:
        with pytest.raises(T.SwzError):
            T.swz_predict_conflicts(kind, layout)
        return
    model = oracle_model()
    wc, rc = T.swz_predict_conflicts(kind, layout)
    ow = sum(O.conflict_report(a, w, model.for_access(w, True))[0] for a, w in T.swz_kernel_accesses(kind, layout, None, 1))
    orc = sum(O.conflict_report(a, w, model.for_access(w, False))[0]
              for a, w in T.swz_kernel_accesses(kind, layout, None, 0))
    assert (wc, rc) == (ow, orc)


@pytest.mark.parametrize("kind", list(KIND_GEOM))
def test_chooser_matches_oracle_chooser(kind):
    """Same bank model, same lane patterns: the oracle's chooser (pinned to
    the pages' own choices under their bank model) picks the same triple,
    and it is predicted conflict-free."""
    esz, tr, tc, _ = KIND_GEOM[kind]
    vec = 4 if kind in NARROW else {4: 4, 2: 16, 1: 8}[esz]
    (b, m, s), cyc = O.choose(esz, vec, tr, tc, restated_accesses(kind, 1), restated_accesses(kind, 0), oracle_model())
    assert T.swz_choose(esz, vec, tr, tc, kind) == (b, m, s)
    assert cyc == 0
    assert T.swz_predict_conflicts(kind, "swizzle") == (0, 0)


def test_model_matches_measured_geometry():
    """The built-in model is the one the LDS microbenchmark measured."""
    m = T.swz_bank_model_get()
    assert (m[("read", 4)]["n_banks"], m[("read", 8)]["n_banks"], m[("read", 16)]["n_banks"]) == (32, 64, 64)
    assert all(m[("write", w)]["n_banks"] == 32 for w in (4, 8, 16))
    assert all(m[(d, w)]["bank_bytes"] == 4 for d in ("read", "write") for w in (4, 8, 16))
    assert m[("read", 4)]["phase"] == [l // 32 for l in range(64)]
    ph = m[("read", 16)]["phase"]
    first = [0, 1, 2, 3, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25, 26, 27]
    assert sorted(l for l in range(64) if ph[l] == ph[0]) == first
    assert len(set(ph)) == 4
    # writes: 32 contiguous lanes for 4-byte writes (the conflict counter's
    # phases), 16 for 8-byte and 8 for 16-byte ones
    assert m[("write", 4)]["phase"] == [l // 32 for l in range(64)]
    assert m[("write", 8)]["phase"] == [l // 16 for l in range(64)]
    assert m[("write", 16)]["phase"] == [l // 8 for l in range(64)]


# ------------------------------------------------- direct HBM -> LDS fill


def test_direct_validation():
    f = lib.swz_convert_layout
    D = T.LAYOUT_SWIZZLE_DIRECT
    # row pitch of 100 bf16 elements (200 bytes) is not a multiple of 16
    assert f(A, B, 2, 64, 100, 2, D, T.READ_B128_8X8, None, None) == EUNSUP
    assert f(A, B, 1, 60, 64, 2, D, T.READ_B64_4X4, None, None) == EUNSUP  # output pitch
    assert f(A + 4, B, 1, 64, 64, 4, D, T.READ_SCALAR_COL, None, None) == EUNSUP  # pointer
    # the same arguments are fine for the register fill (no launch: empty batch)
    assert f(A, B, 0, 64, 100, 2, 0, T.READ_B128_8X8, None, None) == T.SWZ_OK
    # S < B: the swizzle is not its own inverse, the direct fill cannot place it
    assert f(A, B, 1, 64, 64, 2, D, T.READ_B64_4X4, ctypes.byref(P(3, 3, 2)), None) == EINVAL
    assert lib.swz_stage_operand(A, B, 16, 32, 2, 0, D, ctypes.byref(P(4, 3, 2)), None) == EINVAL
    with pytest.raises(T.SwzError):
        T.swz_plan(0, 64, 100, 2, "direct", T.READ_B128_8X8)
    p = T.swz_plan(0, 8192, 8192, 2, "direct", T.READ_B64_4X4)
    assert p["layout"] == T.LAYOUT_SWIZZLE_DIRECT and p["vec_bytes"] == 16 and p["pad_elems"] == 0
    assert p["params"] == T.swz_plan(0, 8192, 8192, 2, "swizzle", T.READ_B64_4X4)["params"]
    assert T.swz_plan(0, 4096, 4096, 4, "direct")["vec_bytes"] == 4


@pytest.mark.parametrize("kind", list(KIND_GEOM))
def test_direct_fill_writes_lane_linear_and_reads_like_swizzle(kind):
    esz, tr, tc, _ = KIND_GEOM[kind]
    nt = threads_of(kind)
    vb = 16 if esz == 2 and kind not in NARROW else 4
    loads = tr * tc * esz // vb // nt
    acc = T.swz_kernel_accesses(kind, "direct", None, 1)
    assert len(acc) == loads * nt // 64
    n = 0
    for w in range(nt // 64):
        for j in range(loads):
            addrs, width = acc[n]
            assert width == vb
            assert addrs == [vb * (64 * w + l + nt * j) for l in range(64)]
            n += 1
    assert T.swz_kernel_accesses(kind, "direct", None, 0) == T.swz_kernel_accesses(kind, "swizzle", None, 0)
    assert T.swz_predict_conflicts(kind, "direct") == (0, 0)


@pytest.mark.parametrize("kind", list(KIND_GEOM))
def test_direct_fill_places_every_element_where_swizzle_does(kind):
    """Reading of the direct fill: the lane filling LDS slot p fetches tile
    element swizzle(p).  With the oracle's swizzle and tile offset, that
    element's swizzled-layout address is p again, for every slot of the tile
    and for every S >= B the chooser could emit -- so the fill reproduces
    the swizzled tile exactly, and covers each element once."""
    esz, tr, tc, _ = KIND_GEOM[kind]
    vb = 16 if esz == 2 and kind not in NARROW else 4  # bytes per direct load
    epl = vb // esz
    # M keeps a load's elements together (and, for the 8-bit kind, its 8-byte LDS writes)
    m_min = (epl.bit_length() - 1) if kind in NARROW or esz != 1 else 3
    log_tile = (tr * tc).bit_length() - 1
    for B, M, S in [(b, m, s) for b in range(1, 6) for m in (m_min, m_min + 1) for s in range(b, 8)
                    if m + b <= log_tile]:
        fetched = []
        for p in range(0, tr * tc, epl):
            e = O.swizzle(p, B, M, S)
            assert e % epl == 0  # a 16-byte slot stays one run of 8 elements
            r, c = divmod(e, tc)
            assert O.tile_offset(r, c, tc, "swizzle", (B, M, S)) == p
            fetched.append(e)
        assert sorted(fetched) == list(range(0, tr * tc, epl))


def test_gemm_validation():
    f = lib.swz_gemm_frag
    assert f(A, B, C, 24, 32, 32, 0, None) == EINVAL  # m not a multiple of 16
    assert f(A, B, C, 32, 24, 32, 0, None) == EINVAL  # n
    assert f(A, B, C, 32, 32, 48, 0, None) == EINVAL  # k not a multiple of 32
    assert f(A, B, C, 32, 32, 32, 1, None) == EINVAL  # fragment kind
    assert f(A + 8, B, C, 32, 32, 32, 0, None) == EINVAL  # alignment
    assert f(A, B, None, 32, 32, 32, 0, None) == EINVAL
    assert f(A, B, A + 64, 32, 32, 32, 0, None) == EINVAL  # C overlaps A's fragments
    assert f(A, B, C, -16, 32, 32, 0, None) == EINVAL
    assert f(A, B, C, 0, 32, 32, 0, None) == T.SWZ_OK  # empty: no launch
    assert f(A, B, C, 1 << 40, 1 << 40, 32, 0, None) == EINVAL  # size overflow



def test_narrow_kind_validation():
    f = lib.swz_convert_layout
    # a narrow kind takes exactly its row width; AUTO picks it for 1, 2, 4, 8, 16 columns
    assert f(A, B, 1, 256, 12, 4, 0, T.READ_NARROW8, None, None) == EINVAL
    assert f(A, B, 1, 256, 8, 2, 0, T.READ_NARROW8, None, None) == EINVAL  # 4-byte elements only
    for c, kind in ((1, T.READ_NARROW1), (2, T.READ_NARROW2), (4, T.READ_NARROW4), (8, T.READ_NARROW8),
                    (16, T.READ_NARROW16)):
        p = T.swz_plan(0, 1000, c, 4, "swizzle")
        assert p["read_kind"] == kind and p["tile"] == (1024 // c, c) and p["lds_bytes"] == 4096
    for c in (32, 64, 96, 120, 127, 128, 129, 200):  # from 96 columns on: fuller last tiles keep the tile kind
        assert T.swz_plan(0, 1000, c, 4, "swizzle")["read_kind"] == T.READ_SCALAR_COL
    for c in (3, 12, 17, 48, 63, 65, 95, 97, 100, 115):  # other widths up to 128 columns: flat whole rows
        assert T.swz_plan(0, 1000, c, 4, "swizzle")["read_kind"] == T.READ_ROWS
    # 2- and 1-byte elements: whole-row tiles for rows of up to 64 bytes
    for esz, kinds in ((2, NARROW2), (1, NARROW1)):
        for i, kind in enumerate(kinds):
            c = 1 << i
            p = T.swz_plan(0, 1024, c, esz, "swizzle")
            cb = min(c, 4 // esz) if esz == 1 or c in (1, 32) else 1  # columns per lane block: the tile is 16 * threads * cb bytes
            tb = 16 * p["threads"] * cb
            assert p["read_kind"] == kind and p["tile"] == (tb // esz // c, c) and p["lds_bytes"] == tb
            assert p["vec_bytes"] == 4 and p["params"][1] == {2: 1, 1: 2}[esz]
        assert f(A, B, 1, 256, 2 * c, esz, 0, kinds[-1], None, None) == EINVAL  # width differs
        assert f(A, B, 1, 256, c, 6 - esz, 0, kinds[-1], None, None) == EINVAL  # element size differs
    assert T.swz_plan(0, 1000, 64, 2)["read_kind"] == T.READ_B64_TR16
    assert T.swz_plan(0, 1000, 48, 2)["read_kind"] == T.READ_ROWS
    assert T.swz_plan(0, 1000, 24, 2)["read_kind"] == T.READ_ROWS
    assert T.swz_plan(0, 1000, 63, 1)["read_kind"] == T.READ_ROWS
    assert T.swz_plan(0, 1000, 100, 2)["read_kind"] == T.READ_ROWS
    assert T.swz_plan(0, 1000, 129, 2)["read_kind"] == T.READ_B64_TR16
    assert T.swz_plan(0, 1000, 127, 1)["read_kind"] == T.READ_ROWS
    assert T.swz_plan(0, 1000, 129, 1)["read_kind"] == T.READ_B64_TR8
    assert T.swz_plan(0, 1000, 128, 2)["read_kind"] == T.READ_B128_8X8
    assert T.swz_plan(0, 1000, 256, 1)["read_kind"] == T.READ_B64_TR8
    assert T.swz_plan(0, 1000, 128, 1)["read_kind"] == T.READ_B64_TR8
    # rows under one 4-byte LDS store get no padded layout
    for kind, c, esz in ((T.READ_HNARROW1, 1, 2), (T.READ_BNARROW1, 1, 1), (T.READ_BNARROW2, 2, 1)):
        assert f(A, B, 1, 256, c, esz, T.LAYOUT_PAD, kind, None, None) == EUNSUP
    assert T.swz_plan(0, 256, 4, 1, "pad")["pad_elems"] == 4 and T.swz_plan(0, 256, 2, 2, "pad")["pad_elems"] == 2
    # M too small to keep a 4-byte LDS write whole
    assert f(A, B, 1, 256, 8, 2, 0, T.READ_HNARROW8, ctypes.byref(P(4, 0, 5)), None) == EINVAL
    assert f(A, B, 1, 256, 8, 1, 0, T.READ_BNARROW8, ctypes.byref(P(4, 1, 5)), None) == EINVAL
    # whole-row tiles need only the output pitch aligned for the vector path
    assert T.swz_plan(0, 4096, 1, 4, "swizzle")["aligned"] and T.swz_plan(0, 4096, 2, 4, "direct")["aligned"]
    assert not T.swz_plan(0, 4093, 8, 4, "swizzle", T.READ_NARROW8)["aligned"]
    # ... and where the output rows rule out 16-byte vectors, AUTO takes flat rows for every fp32
    # width, 2-byte widths of 8 to 32 and bytes x 64 (the narrow kinds would go element by element)
    for esz, c, kind in ((4, 1, T.READ_ROWS), (4, 16, T.READ_ROWS), (2, 4, T.READ_HNARROW4), (2, 8, T.READ_ROWS),
                         (2, 32, T.READ_ROWS), (1, 32, T.READ_BNARROW32), (1, 64, T.READ_ROWS)):
        assert T.swz_plan(0, 4093, c, esz, "swizzle")["read_kind"] == kind, (esz, c)
        assert T.swz_plan(0, 4096, c, esz, "swizzle")["read_kind"] != T.READ_ROWS, (esz, c)  # aligned rows
    assert T.swz_get_tile_order(1, 4093, 8, 4) == T.ORDER_DIAGONAL  # resolves to the flat-row kind too
    # the flat-row kind has no padded or direct layout: AUTO keeps the tile and narrow kinds for those
    assert T.swz_plan(0, 1000, 3, 4, "pad")["read_kind"] == T.READ_SCALAR_COL
    assert T.swz_plan(0, 1000, 100, 2, "pad")["read_kind"] == T.READ_B128_8X8
    assert T.swz_plan(0, 4093, 8, 4, "pad")["read_kind"] == T.READ_NARROW8
    assert T.swz_plan(0, 1024, 12, 4, "direct")["read_kind"] == T.READ_SCALAR_COL  # 16-byte pitches: direct fill
    assert f(A, B, 0, 1000, 3, 4, T.LAYOUT_PAD, T.READ_AUTO, None, None) == T.SWZ_OK  # nothing to move: no launch
    assert f(A, B, 1, 4093, 8, 4, T.LAYOUT_SWIZZLE_DIRECT, T.READ_NARROW8, None, None) == EUNSUP
    # the flat-offset swizzle spans rows: Swizzle<5,0,5> on a 128x8 tile XORs
    # row bits 2-6 into the element bits (the pages' int num[32][8] example)
    assert T.swz_choose(4, 4, 128, 8, T.READ_NARROW8) == (5, 0, 5)


def test_fused_gemm_bf16_validation():
    f = lib.swz_gemm_ex
    assert f(A, B, C, 32, 32, 32, 0, None, 2, None) == EINVAL  # no such result type
    assert f(A, B, C, 24, 32, 32, 0, None, T.C_BF16, None) == EINVAL  # m not a multiple of 16
    assert f(A, B, C, 32, 32, 32, T.LAYOUT_PAD, None, T.C_BF16, None) == EUNSUP
    assert f(A, B, A + 1024, 32, 32, 32, 0, None, T.C_BF16, None) == EINVAL  # C overlaps A
    assert f(A, B, C + 8, 32, 32, 32, 0, None, T.C_BF16, None) == EINVAL  # alignment
    assert f(A, B, C, 0, 32, 32, 0, None, T.C_BF16, None) == T.SWZ_OK  # empty: no launch


def test_fused_gemm_validation():
    f = lib.swz_gemm
    assert f(A, B, C, 24, 32, 32, 0, None, None) == EINVAL  # m not a multiple of 16
    assert f(A, B, C, 32, 24, 32, 0, None, None) == EINVAL  # n
    assert f(A, B, C, 32, 32, 48, 0, None, None) == EINVAL  # k not a multiple of 32
    assert f(A + 8, B, C, 32, 32, 32, 0, None, None) == EINVAL  # alignment
    assert f(A, B, None, 32, 32, 32, 0, None, None) == EINVAL
    assert f(A, B, A + 64, 32, 32, 32, 0, None, None) == EINVAL  # C overlaps A
    assert f(A, B, C, -16, 32, 32, 0, None, None) == EINVAL
    assert f(A, B, C, 1 << 40, 1 << 40, 32, 0, None, None) == EINVAL  # size overflow
    assert f(A, B, C, 32, 32, 32, 7, None, None) == EINVAL  # layout
    assert f(A, B, C, 32, 32, 32, T.LAYOUT_PAD, None, None) == EUNSUP
    # |S| < B: the direct fill cannot place it; a field leaving the 64x64 tile
    assert f(A, B, C, 32, 32, 32, 0, ctypes.byref(P(4, 3, 2)), None) == EINVAL
    assert f(A, B, C, 32, 32, 32, 0, ctypes.byref(P(4, 3, -8)), None) == EINVAL
    for layout in (0, T.LAYOUT_PLAIN, T.LAYOUT_SWIZZLE_DIRECT):
        assert f(A, B, C, 0, 32, 32, layout, None, None) == T.SWZ_OK  # empty: no launch


def test_negative_shift_validation():
    assert lib.swz_map(A, B, 16, P(5, 20, -8), None) == EINVAL  # fields leave 32 bits
    f = lib.swz_convert_layout
    # the changed field [M+|S|, M+|S|+B) = [3+6, 13) leaves the 64x64 tile (12 bits)
    assert f(A, B, 1, 64, 64, 2, 0, T.READ_B64_4X4, ctypes.byref(P(4, 3, -6)), None) == EINVAL
    # |S| < B cannot be placed by the direct fill
    assert f(A, B, 1, 64, 64, 2, T.LAYOUT_SWIZZLE_DIRECT, T.READ_B64_4X4, ctypes.byref(P(3, 3, -2)), None) == EINVAL
    p = T.swz_plan(0, 64, 64, 2, "swizzle", T.READ_B64_4X4, (3, 3, -4))
    assert p["params"] == (3, 3, -4)
    w, r = T.swz_predict_conflicts(T.READ_B64_4X4, "swizzle", (3, 3, -4))
    assert w >= 0 and r >= 0


@pytest.mark.parametrize("kind", list(KIND_GEOM))
def test_kernel_accesses_negative_shift(kind):
    esz, tr, tc, pad = KIND_GEOM[kind]
    params = (3, 0, -4) if esz == 4 else (3, 3, -4)
    for write in (1, 0):
        lib_acc = T.swz_kernel_accesses(kind, "swizzle", params, write)
        mine = restated_accesses(kind, write)
        for (addrs, width), (coords, w2) in zip(lib_acc, mine):
            expect = [esz * int(O.swizzle_signed(a // esz, *params)) for a in
                      O.access_addresses(coords, width // esz, tc, esz, "plain", (0, 0, 0), 0)]
            assert addrs == expect


def test_fold_matches_oracle():
    rng = np.random.default_rng(22)
    for _ in range(500):
        B = int(rng.integers(1, 6))
        M = int(rng.integers(0, 6))
        S = int(rng.choice([-1, 1])) * int(rng.integers(1, 9))
        active = int(rng.integers(0, 1 << 20))
        base = int(rng.integers(0, 1 << 24)) & ~active
        coll, fb, strides = T.swz_fold((B, M, S), base, active)
        assert coll == O.fold_collision(active, B, M, S)
        if coll == 0:
            ob, ostr = O.fold_strides(base, active, B, M, S)
            assert fb == ob and strides == ostr
        else:
            assert fb is None


def test_fold_validation():
    c = ctypes.c_uint32()
    assert lib.swz_fold(ctypes.byref(P(3, 0, 3)), 1, 1, ctypes.byref(c), None, None) == EINVAL  # base & active
    assert lib.swz_fold(ctypes.byref(P(3, 20, 12)), 0, 1, ctypes.byref(c), None, None) == EINVAL
    assert lib.swz_fold(ctypes.byref(P(3, 0, 3)), 0, 1, None, None, None) == EINVAL
    # the 32x32 fp32 tile's (5,0,5) over a whole tile collides; over one row it folds
    assert T.swz_fold((5, 0, 5), 0, 1023)[1] is None
    coll, fb, strides = T.swz_fold((5, 0, 5), 7 * 32, 31)  # row 7: column bits only
    assert coll == 0 and fb == 7 * 32 + 7
    assert strides == {b: (-(1 << b) if (7 >> b) & 1 else (1 << b)) for b in range(5)}


def test_auto_read_kind_picks_the_kernels_the_workloads_are_timed_with():
    """SWZ_READ_AUTO stands for a call without the read-kind argument: for the
    workloads' shapes it resolves to the kernels the benchmark times (fp32
    4096^2: 4-byte column reads; fp16 8192^2: 8-byte reads of 4x4 blocks;
    bf16 [64,4096,128]: 128-wide rows, 16-byte reads of 8x8 blocks; staging:
    the operand-fragment pattern)."""
    cases = [
        (0, 4096, 4096, 4, T.READ_SCALAR_COL),
        (0, 8192, 8192, 2, T.READ_B64_4X4),
        (0, 1 << 18, 256, 2, T.READ_B64_TR16),  # the widest 16-bit rows that keep transpose reads
        (0, 4096, 320, 2, T.READ_B64_4X4),
        (0, 4096, 128, 2, T.READ_B128_8X8),
        (1, 8192, 4096, 2, T.READ_MFMA_16X16X32),
        (0, 8192, 8192, 1, T.READ_B64_TR8),
        (0, 1 << 21, 8, 4, T.READ_NARROW8),
    ]
    for op, rows, cols, esz, kind in cases:
        for layout in ("swizzle", "pad", "plain"):
            assert T.swz_plan(op, rows, cols, esz, layout, T.READ_AUTO)["read_kind"] == kind, (rows, cols, esz)


def test_rows_kind_plan_and_validation():
    """Flat whole-row tiles (SWZ_READ_ROWS): any width up to 128 columns, as
    many rows as fit in 16 KiB (32 KiB and 512 threads above 64 columns) in
    groups of 64 lane-words (4 bytes of rows each) plus 64 bytes' worth of
    halo rows in LDS, a word-offset swizzle
    for even widths, SWIZZLE and PLAIN layouts only; an explicit swizzle
    must have M = 0, B <= 10 and B <= S <= 11."""
    f = lib.swz_convert_layout
    for esz, cmax in ((4, 128), (2, 128), (1, 128)):
        group = 64 * (4 // esz)
        for c in range(1, cmax + 1):
            p = T.swz_plan(0, 100000, c, esz, "swizzle", T.READ_ROWS)
            tb, nt = (16384, 256) if c <= 64 else (32768, 512)  # tile bytes and threads
            tr = tb // (c * esz) // group * group
            assert p["read_kind"] == T.READ_ROWS and p["tile"] == (tr, c)
            assert p["lds_bytes"] == (tr + 64 // esz) * c * esz <= tb + tb // 4
            B, M, S = p["params"]
            if c % 2:  # odd widths read conflict-free unswizzled
                assert (B, M, S) == (0, 0, 0), (c, p["params"])
            elif c % 4 == 0:  # a swizzle of word offsets whose source lies above the bank bits
                assert B >= 2 and M == 0 and B <= S <= 11, (c, p["params"])
            else:  # the search's pick, whichever it is, a valid word-offset swizzle or none
                assert M == 0 and (B == 0 or B <= S <= 11), (c, p["params"])
            assert p["pad_elems"] == 0 and p["threads"] == nt and p["aligned"]
            assert tr >= group and tr * c * esz <= tb
            plain = T.swz_plan(0, 100000, c, esz, "plain", T.READ_ROWS)
            assert plain["tile"] == (tr, c) and plain["params"] == (0, 0, 0)
        assert f(A, B, 1, 256, cmax + 1, esz, 0, T.READ_ROWS, None, None) == EINVAL  # wider than 128 columns
        assert f(A, B, 1, 256, 3, esz, T.LAYOUT_PAD, T.READ_ROWS, None, None) == EUNSUP
        assert f(A, B, 1, 256, 3, esz, T.LAYOUT_SWIZZLE_DIRECT, T.READ_ROWS, None, None) == EUNSUP
        assert f(A, B, 1, 256, 3, esz, 0, T.READ_ROWS, ctypes.byref(P(3, 2, 3)), None) == EINVAL  # M != 0
        assert f(A, B, 1, 256, 3, esz, 0, T.READ_ROWS, ctypes.byref(P(3, 0, 2)), None) == EINVAL  # S < B
        assert f(A, B, 1, 256, 3, esz, 0, T.READ_ROWS, ctypes.byref(P(1, 0, 12)), None) == EINVAL  # S past the tile
        assert f(A, B, 1, 256, 3, esz, 0, T.READ_ROWS, ctypes.byref(P(11, 0, 11)), None) == EINVAL  # B past the LDS
        assert T.swz_plan(0, 256, 6, esz, "swizzle", T.READ_ROWS, (10, 0, 11))["params"] == (10, 0, 11)
        assert T.swz_plan(0, 256, 6, esz, "swizzle", T.READ_ROWS, (2, 0, 7))["params"] == (2, 0, 7)
        assert T.swz_plan(0, 256, 3, esz, "swizzle", T.READ_ROWS, (0, 0, 0))["read_kind"] == T.READ_ROWS
        assert T.swz_plan(0, 257, 3, esz, "swizzle", T.READ_ROWS)["aligned"]  # any pitch takes the same kernel
    assert lib.swz_choose(4, 4, 32, 32, T.READ_ROWS, ctypes.byref(P())) == EINVAL  # not a swizzled kind
