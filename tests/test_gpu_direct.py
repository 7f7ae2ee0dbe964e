"""Bit-exact parity of the direct HBM -> LDS fill (SWZ_LAYOUT_SWIZZLE_DIRECT)
against the CPU oracle (needs a GPU).

The direct fill changes how the tile reaches LDS, not what the call
computes: the expected values are the oracle's transposes and fragments.
Shapes keep 16-byte row pitches (the layout's precondition) and still cover
whole tiles, ragged edge tiles, single rows and columns, and empty inputs.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W

import torch  # noqa: E402  (hard imports: a GPU run without them fails, never skips)

import tiled_movement_amd as T  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SIGNED = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32, np.dtype(np.uint8): np.uint8}


def to_dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(SIGNED[a.dtype])).to(DEV)


def from_dev(t, like):
    return t.cpu().numpy().view(like.dtype)


def announce(*what):
    print("case:", *what, flush=True)


KINDS = [
    (T.READ_SCALAR_COL, 4, 32, 32, W.fp32_matrix, 4),
    (T.READ_B64_4X4, 2, 64, 64, W.fp16_matrix, 8),
    (T.READ_B128_8X8, 2, 64, 128, lambda r, c, seed: W.bf16_tensor((r, c), seed=seed), 8),
    (T.READ_B64_TR16, 2, 64, 64, W.fp16_matrix, 8),
    (T.READ_B64_TR8, 1, 128, 128, W.u8_matrix, 16),
]


def direct_shapes(tr, tc, q):
    """q: the element count of 16 bytes, so every pitch stays 16-byte aligned."""
    return [
        (3 * tr, 2 * tc),
        (2 * tr + q, 3 * tc + 3 * q),  # ragged edge tiles both ways
        (3 * tr + q, 2 * tc + q),  # an odd count of whole tile rows, then a ragged one
        (tr - q, tc + q),
        (q, q),
        (q, 5 * tc + q),
        (4 * tr + q, q),
        (0, q),
        (q, 0),
    ]


def check(a, esz, kind, params=None):
    rows, cols = a.shape
    src = to_dev(a)
    dst = torch.empty((cols, rows), dtype=src.dtype, device=DEV)
    T.swz_transpose(src, dst, rows, cols, esz, "direct", kind, params)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dst, a), O.transpose(a)), (a.shape, kind, params)


@pytest.mark.parametrize("kind,esz,tr,tc,gen,q", KINDS)
def test_direct_transpose_shapes(kind, esz, tr, tc, gen, q):
    for seed, (rows, cols) in enumerate(direct_shapes(tr, tc, q)):
        announce("direct transpose", kind, rows, cols)
        check(gen(rows, cols, seed=seed), esz, kind)


@pytest.mark.parametrize("kind,esz,tr,tc,gen,q", KINDS)
def test_direct_transpose_any_involutive_swizzle(kind, esz, tr, tc, gen, q):
    rows, cols = 2 * tr + q, 2 * tc + q
    a = gen(rows, cols, seed=14)
    m_min = 0 if esz == 4 else 3  # 1-byte: the swizzle keeps 8-byte runs (M >= 3)
    log_tile = (tr * tc).bit_length() - 1
    triples = [(B, M, S) for B in range(0, 6) for M in range(m_min, 6) for S in range(max(B, 1), 9)
               if M + B <= log_tile]
    rng = np.random.default_rng(100 + kind)
    for idx in rng.choice(len(triples), size=min(12, len(triples)), replace=False):
        announce("direct params", kind, triples[idx])
        check(a, esz, kind, triples[idx])


def test_direct_convert_batches():
    cases = [
        (T.READ_B128_8X8, 2, W.bf16_tensor((3, 200, 128), seed=15)),
        (T.READ_B128_8X8, 2, W.bf16_tensor((2, 64, 96), seed=16)),
        (T.READ_B64_4X4, 2, W.bf16_tensor((2, 72, 136), seed=17)),
        (T.READ_SCALAR_COL, 4, W.fp32_matrix(3 * 40, 52, seed=18).reshape(3, 40, 52)),
        # 2 x 2 stacked fp32 blocks with a whole tile row and column left over
        (T.READ_SCALAR_COL, 4, W.fp32_matrix(2 * 100, 104, seed=24).reshape(2, 100, 104)),
    ]
    for kind, esz, a in cases:
        announce("direct convert", kind, a.shape)
        b, r, c = a.shape
        src = to_dev(a)
        dst = torch.empty((b, c, r), dtype=src.dtype, device=DEV)
        T.swz_convert_layout(src, dst, b, r, c, esz, "direct", kind)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dst, a), O.convert_layout(a))


def test_direct_stage_operand_shapes():
    for mn, k in [(16, 32), (256, 64), (272, 96), (512, 512), (48, 608)]:
        a, bt = W.bf16_operands(mn, mn, k, seed=mn + k + 1)
        for op in (a, bt):
            announce("direct stage", mn, k)
            src = to_dev(op)
            frag = torch.empty(op.size, dtype=src.dtype, device=DEV)
            T.swz_stage_operand(src, frag, mn, k, layout="direct")
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(frag, op), O.stage_operand(op).reshape(-1)), (mn, k)


def test_direct_stage_operand_any_involutive_swizzle():
    # k = 320: four whole k tiles in one stacked workgroup, a fifth in a block of its own
    a, _ = W.bf16_operands(272, 16, 320, seed=19)
    src = to_dev(a)
    ref = O.stage_operand(a).reshape(-1)
    for p in [(0, 3, 1), (3, 3, 3), (3, 3, 4), (4, 3, 4), (2, 4, 7), (5, 3, 6), (1, 3, 1)]:
        announce("direct stage params", p)
        frag = torch.empty(a.size, dtype=src.dtype, device=DEV)
        T.swz_stage_operand(src, frag, 272, 320, layout="direct", params=p)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(frag, a), ref), p


def test_direct_full_fp32_4096():
    announce("direct full fp32 4096")
    check(W.fp32_matrix(4096, 4096, seed=0), 4, T.READ_SCALAR_COL)


def test_direct_full_fp16_8192():
    announce("direct full fp16 8192")
    check(W.fp16_matrix(8192, 8192, seed=0), 2, T.READ_B64_4X4)


def test_direct_full_fp16_8192_transpose_read():
    announce("direct full fp16 8192 transpose read")
    check(W.fp16_matrix(8192, 8192, seed=0), 2, T.READ_B64_TR16)


def test_direct_full_u8_8192_transpose_read():
    announce("direct full u8 8192")
    check(W.u8_matrix(8192, 8192, seed=0), 1, T.READ_B64_TR8)


def test_direct_full_bf16_convert():
    announce("direct full bf16 convert")
    a = W.bf16_tensor((64, 4096, 128), seed=0)
    src = to_dev(a)
    dst = torch.empty((64, 128, 4096), dtype=src.dtype, device=DEV)
    T.swz_convert_layout(src, dst, 64, 4096, 128, 2, "direct", T.READ_B128_8X8)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dst, a), O.convert_layout(a))


def test_direct_full_operand_staging():
    announce("direct full staging")
    a, bt = W.bf16_operands(8192, 8192, 4096, seed=0)
    for op in (a, bt):
        src = to_dev(op)
        frag = torch.empty(op.size, dtype=src.dtype, device=DEV)
        T.swz_stage_operand(src, frag, op.shape[0], op.shape[1], layout="direct")
        torch.cuda.synchronize()
        got = from_dev(frag, op).reshape(op.shape[0] // 16, op.shape[1] // 32, 64, 8)
        assert np.array_equal(got, O.stage_operand(op))


def test_direct_rejects_unaligned_pitch_before_launch():
    a = W.bf16_tensor((2, 64, 100), seed=20)
    src = to_dev(a)
    dst = torch.empty((2, 100, 64), dtype=src.dtype, device=DEV)
    with pytest.raises(T.SwzError):
        T.swz_convert_layout(src, dst, 2, 64, 100, 2, "direct", T.READ_B128_8X8)
