"""The consumer of the staged fragments (needs a GPU): swz_stage_operand
for A and for B^T, then swz_gemm_frag, against the oracle's fp64 product.

Integer-valued operands make every partial sum exact in fp32, so those
cases must match bit for bit; random operands must stay within the
oracle's bound for fp32 accumulation in 32-wide chunks (with a factor of 2
of margin).
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


def int_bf16(shape, seed, lo=-2, hi=3):
    v = np.random.default_rng(seed).integers(lo, hi, size=shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def gemm_on_gpu(a, bt, layout="swizzle"):
    m, k = a.shape
    n = bt.shape[0]
    fa = torch.empty(a.size, dtype=torch.int16, device=DEV)
    fb = torch.empty(bt.size, dtype=torch.int16, device=DEV)
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    if k:
        T.swz_stage_operand(torch.from_numpy(a.view(np.int16)).to(DEV), fa, m, k, layout=layout)
        T.swz_stage_operand(torch.from_numpy(bt.view(np.int16)).to(DEV), fb, n, k, layout=layout)
    T.swz_gemm_frag(fa, fb, c, m, n, k)
    torch.cuda.synchronize()
    return c.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,n,k", [(16, 16, 32), (256, 256, 64), (272, 400, 96), (512, 256, 4096), (48, 784, 160)])
def test_integer_operands_exact(m, n, k):
    announce("gemm exact", m, n, k)
    a, bt = int_bf16((m, k), m + k), int_bf16((n, k), n + 3 * k)
    got = gemm_on_gpu(a, bt)
    assert np.array_equal(got, O.gemm_bf16(a, bt))


def test_fragments_from_every_layout_give_the_same_product():
    a, bt = int_bf16((272, 96), 1), int_bf16((144, 96), 2)
    ref = O.gemm_bf16(a, bt)
    for layout in ("swizzle", "pad", "plain", "direct"):
        announce("gemm after staging", layout)
        assert np.array_equal(gemm_on_gpu(a, bt, layout), ref)


def test_k_zero_writes_zeros():
    announce("gemm k=0")
    got = gemm_on_gpu(np.zeros((32, 0), np.uint16), np.zeros((48, 0), np.uint16))
    assert got.shape == (32, 48) and np.all(got == 0)


def test_random_operands_within_fp32_bound():
    announce("gemm random 512x768x4096")
    a, bt = W.bf16_operands(512, 768, 4096, seed=5, std=1.0)
    got = gemm_on_gpu(a, bt)
    err = np.abs(got - O.gemm_bf16(a, bt))
    assert np.all(err <= 2 * O.gemm_error_bound(a, bt))


def test_full_size_sampled_rows():
    """A [8192 x 4096] and B^T [8192 x 4096] (the staging workload's
    operands): rows sampled across the first, middle and last 256-row tiles
    are compared with the oracle within the bound."""
    announce("gemm full 8192x8192x4096")
    a, bt = W.bf16_operands(8192, 8192, 4096, seed=0)
    got_dev = None
    fa = torch.empty(a.size, dtype=torch.int16, device=DEV)
    fb = torch.empty(bt.size, dtype=torch.int16, device=DEV)
    T.swz_stage_operand(torch.from_numpy(a.view(np.int16)).to(DEV), fa, 8192, 4096)
    T.swz_stage_operand(torch.from_numpy(bt.view(np.int16)).to(DEV), fb, 8192, 4096)
    c = torch.empty((8192, 8192), dtype=torch.float32, device=DEV)
    T.swz_gemm_frag(fa, fb, c, 8192, 8192, 4096)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 15, 16, 255, 256, 4095, 4100, 8191, 8190, 7936, 3333])
    got_dev = c[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    ref = O.gemm_bf16(a[rows], bt)
    bound = O.gemm_error_bound(a[rows], bt)
    assert np.all(np.abs(got_dev - ref) <= 2 * bound)


# ------------------------------------------ swz_gemm: staging inside the GEMM
def fused_on_gpu(a, bt, layout="swizzle", params=None):
    m, k = a.shape
    n = bt.shape[0]
    c = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    da = torch.from_numpy(a.view(np.int16)).to(DEV)
    db = torch.from_numpy(bt.view(np.int16)).to(DEV)
    T.swz_gemm(da, db, c, m, n, k, layout=layout, params=params)
    torch.cuda.synchronize()
    return c.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,n,k", [(16, 16, 32), (256, 256, 64), (272, 400, 96), (512, 256, 4096), (48, 784, 160),
                                   (784, 48, 32), (512, 512, 2080)])
@pytest.mark.parametrize("layout", ["swizzle", "plain"])
def test_fused_integer_operands_exact(m, n, k, layout):
    announce("fused gemm exact", layout, m, n, k)
    a, bt = int_bf16((m, k), m + k + 7), int_bf16((n, k), n + 3 * k + 7)
    assert np.array_equal(fused_on_gpu(a, bt, layout), O.gemm_bf16(a, bt))


@pytest.mark.parametrize("params", [(4, 3, 4), (4, 3, -4), (3, 3, 3), (2, 3, 5), (0, 0, 0)])
def test_fused_explicit_params_exact(params):
    """Any swizzle the direct fill can place gives the same product: the
    layout only decides where each element sits in LDS."""
    announce("fused gemm params", params)
    a, bt = int_bf16((272, 192), 11), int_bf16((528, 192), 12)
    assert np.array_equal(fused_on_gpu(a, bt, "swizzle", params), O.gemm_bf16(a, bt))


def test_fused_direct_is_swizzle():
    announce("fused gemm direct layout")
    a, bt = int_bf16((256, 128), 13), int_bf16((256, 128), 14)
    assert np.array_equal(fused_on_gpu(a, bt, "direct"), fused_on_gpu(a, bt, "swizzle"))


def test_fused_k_zero_writes_zeros():
    announce("fused gemm k=0")
    got = fused_on_gpu(np.zeros((32, 0), np.uint16), np.zeros((48, 0), np.uint16))
    assert got.shape == (32, 48) and np.all(got == 0)


def test_fused_equals_fragment_path_bitwise():
    """Same instruction, same k order: the fused GEMM and the staged-fragment
    GEMM give bit-identical fp32 results on random operands."""
    announce("fused vs fragment 512x768x4096")
    a, bt = W.bf16_operands(512, 768, 4096, seed=5, std=1.0)
    fused = fused_on_gpu(a, bt)
    assert np.array_equal(fused, gemm_on_gpu(a, bt))
    err = np.abs(fused - O.gemm_bf16(a, bt))
    assert np.all(err <= 2 * O.gemm_error_bound(a, bt))


@pytest.mark.parametrize("layout", ["swizzle", "plain"])
def test_fused_full_size_sampled_rows(layout):
    """A [8192 x 4096] row-major and B^T [8192 x 4096] (B column-major) at
    full size: sampled rows within the bound of the oracle's fp64 product."""
    announce("fused gemm full 8192x8192x4096", layout)
    a, bt = W.bf16_operands(8192, 8192, 4096, seed=0)
    c = torch.empty((8192, 8192), dtype=torch.float32, device=DEV)
    T.swz_gemm(torch.from_numpy(a.view(np.int16)).to(DEV), torch.from_numpy(bt.view(np.int16)).to(DEV), c,
               8192, 8192, 4096, layout=layout)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 15, 16, 255, 256, 4095, 4100, 8191, 8190, 7936, 3333])
    got = c[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    ref = O.gemm_bf16(a[rows], bt)
    assert np.all(np.abs(got - ref) <= 2 * O.gemm_error_bound(a[rows], bt))


# ------------------------------------------------- bf16 result (swz_gemm_ex)


def fused_bf16_on_gpu(a, bt, layout="swizzle", params=None):
    m, k = a.shape
    n = bt.shape[0]
    c = torch.full((m, n), -1, dtype=torch.int16, device=DEV)
    da = torch.from_numpy(a.view(np.int16)).to(DEV)
    db = torch.from_numpy(bt.view(np.int16)).to(DEV)
    T.swz_gemm_ex(da, db, c, m, n, k, layout=layout, params=params, c_type=T.C_BF16)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("m,n,k", [(16, 16, 32), (272, 400, 96), (784, 48, 32), (512, 512, 2080)])
@pytest.mark.parametrize("layout", ["swizzle", "plain"])
def test_fused_bf16_result_is_the_rounded_fp32_result(m, n, k, layout):
    """Same accumulation as the fp32 result, then rounded to nearest even:
    bit for bit the oracle's rounding of the fp32 kernel's output, and within
    the fp32 bound plus half a bf16 step of the exact product."""
    announce("fused gemm bf16", m, n, k, layout)
    a, bt = W.bf16_operands(m, n, k, seed=m + n + k, std=1.0)
    c32 = fused_on_gpu(a, bt, layout)
    c16 = fused_bf16_on_gpu(a, bt, layout)
    assert np.array_equal(c16, O.f32_to_bf16_bits(c32.astype(np.float32)))
    exact = O.gemm_bf16(a, bt)
    got = O.bf16_to_f64(c16)
    bound = 2 * O.gemm_error_bound(a, bt)
    assert np.all(np.abs(got - exact) <= bound + 2.0 ** -8 * (np.abs(exact) + bound))


def test_fused_bf16_integer_operands_exact():
    """Integer-valued operands: the fp32 sums are exact, so the bf16 result is
    the oracle's rounding of the exact product."""
    rng = np.random.default_rng(21)
    for m, n, k in [(256, 256, 64), (272, 400, 96), (48, 784, 160)]:
        announce("fused gemm bf16 integers", m, n, k)
        ia = (rng.integers(-3, 4, size=(m, k)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        ib = (rng.integers(-3, 4, size=(n, k)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        c16 = fused_bf16_on_gpu(ia, ib)
        assert np.array_equal(c16, O.f32_to_bf16_bits(O.gemm_bf16(ia, ib).astype(np.float32)))


def test_fused_bf16_k_zero_writes_zeros():
    a = np.zeros((32, 0), dtype=np.uint16)
    bt = np.zeros((48, 0), dtype=np.uint16)
    c = torch.full((32, 48), -1, dtype=torch.int16, device=DEV)
    T.swz_gemm_ex(torch.empty(16, dtype=torch.int16, device=DEV), torch.empty(16, dtype=torch.int16, device=DEV),
                  c, 32, 48, 0, c_type=T.C_BF16)
    torch.cuda.synchronize()
    assert not c.any().item()
    del a, bt


def test_fused_bf16_full_size():
    """A [8192 x 4096], B^T [8192 x 4096]: the whole bf16 result equals the
    fp32 result rounded to nearest even (the library's conversion on the
    GPU, which the oracle's rounding is pinned to), and sampled rows equal
    the oracle's rounding directly."""
    announce("fused gemm bf16 full 8192x8192x4096")
    a, bt = W.bf16_operands(8192, 8192, 4096, seed=0)
    da = torch.from_numpy(a.view(np.int16)).to(DEV)
    db = torch.from_numpy(bt.view(np.int16)).to(DEV)
    c32 = torch.empty((8192, 8192), dtype=torch.float32, device=DEV)
    c16 = torch.empty((8192, 8192), dtype=torch.int16, device=DEV)
    T.swz_gemm(da, db, c32, 8192, 8192, 4096)
    T.swz_gemm_ex(da, db, c16, 8192, 8192, 4096, c_type=T.C_BF16)
    torch.cuda.synchronize()
    assert torch.equal(c16, c32.to(torch.bfloat16).view(torch.int16))
    rows = torch.tensor([0, 17, 4095, 8191], device=DEV)
    got = c16[rows].cpu().numpy().view(np.uint16)
    assert np.array_equal(got, O.f32_to_bf16_bits(c32[rows].cpu().numpy()))
