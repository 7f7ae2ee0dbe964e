"""Pin of the operand-fragment layout against the hardware (needs a GPU).

The pages describe the operand read (ldmatrix / WGMMA) but fix no lane order
for AMD; the oracle's stage_operand takes lane l -> row l % 16, k = 8*(l/16)
.. +7 of a 32-wide k step.  Here the real 16x16x32 bf16 matrix instruction
consumes fragments built by the oracle (and, separately, by the library)
and its result is compared with an fp64 product of the operand blocks, read
back under the instruction's output layout (lane l holds rows
4*(l/16) .. +3 of column l % 16).
"""

import ctypes
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

import torch  # noqa: E402  (hard imports: a GPU run without them fails, never skips)

import tiled_movement_amd as T  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def probe():
    path = os.path.join(HERE, "libhw_probe.so")
    if not os.path.exists(path):
        pytest.fail("tests/libhw_probe.so is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.mfma_probe_16x16x32_bf16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_void_p]
    lib.mfma_probe_16x16x32_bf16.restype = ctypes.c_int
    return lib


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def run_mfma(probe, a_frags, b_frags):
    """a_frags, b_frags: uint16 [n, 64, 8] in lane order -> fp32 [n, 64, 4]."""
    n = a_frags.shape[0]
    a = torch.from_numpy(np.ascontiguousarray(a_frags).view(np.int16)).to(DEV)
    b = torch.from_numpy(np.ascontiguousarray(b_frags).view(np.int16)).to(DEV)
    d = torch.empty((n, 64, 4), dtype=torch.float32, device=DEV)
    rc = probe.mfma_probe_16x16x32_bf16(a.data_ptr(), b.data_ptr(), d.data_ptr(), n,
                                         torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return d.cpu().numpy()


def decode(d):
    """Lane-order outputs [64][4] -> 16x16 matrix (row 4*(l//16)+i, col l%16)."""
    out = np.empty((16, 16))
    for lane in range(64):
        for i in range(4):
            out[4 * (lane // 16) + i, lane % 16] = d[lane, i]
    return out


def check_blocks(probe, a, bt, fa, fb):
    mb, kb = a.shape[0] // 16, a.shape[1] // 32
    nb = bt.shape[0] // 16
    pairs = [(i, n, j) for i in range(mb) for n in range(nb) for j in range(kb)]
    d = run_mfma(probe, np.stack([fa[i, j] for i, n, j in pairs]), np.stack([fb[n, j] for i, n, j in pairs]))
    af, bf = bf16_to_f64(a), bf16_to_f64(bt)
    for g, (i, n, j) in enumerate(pairs):
        ref = af[16 * i:16 * i + 16, 32 * j:32 * j + 32] @ bf[16 * n:16 * n + 16, 32 * j:32 * j + 32].T
        got = decode(d[g])
        scale = np.abs(af[16 * i:16 * i + 16, 32 * j:32 * j + 32]) @ np.abs(bf[16 * n:16 * n + 16, 32 * j:32 * j + 32]).T
        assert np.all(np.abs(got - ref) <= 1e-5 * scale + 1e-30), (i, n, j)


def test_oracle_fragments_feed_the_matrix_instruction(probe):
    a, bt = W.bf16_operands(48, 32, 96, seed=21, std=1.0)
    check_blocks(probe, a, bt, O.stage_operand(a), O.stage_operand(bt))


def test_library_fragments_feed_the_matrix_instruction(probe):
    a, bt = W.bf16_operands(272, 48, 96, seed=22, std=1.0)
    frags = []
    for op in (a, bt):
        src = torch.from_numpy(op.view(np.int16)).to(DEV)
        frag = torch.empty(op.size, dtype=torch.int16, device=DEV)
        T.swz_stage_operand(src, frag, op.shape[0], op.shape[1])
        torch.cuda.synchronize()
        frags.append(frag.cpu().numpy().view(np.uint16).reshape(op.shape[0] // 16, op.shape[1] // 32, 64, 8))
    check_blocks(probe, a[:64], bt, frags[0][:4], frags[1])


def test_a_transposed_fragment_order_would_fail(probe):
    """Control: swapping the roles of row and k-group lanes breaks the product,
    so the check above is sensitive to the lane order."""
    a, bt = W.bf16_operands(16, 16, 32, seed=23, std=1.0)
    fa, fb = O.stage_operand(a), O.stage_operand(bt)
    wrong = fa.reshape(1, 1, 4, 16, 8).transpose(0, 1, 3, 2, 4).reshape(1, 1, 64, 8)
    d = run_mfma(probe, wrong[:, 0], fb[:, 0])
    ref = bf16_to_f64(a) @ bf16_to_f64(bt).T
    assert not np.allclose(decode(d[0]), ref)
